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
//  * data: any int32 x (a residue representative) has the bytes of x XOR 0x00808080 as
//    signed digits with x = sum_b s_b 256^b + K0, K0 = 0x808080 (x + 2^31 is the unsigned
//    word x XOR 0x80000000, whose bytes minus 128 are the digits; 128 * 0x01010101 - 2^31
//    is K0), so no value needs reducing to [0, p) before it is split;
//  * matrices: F^(b) = 256^b F mod p (precomputed) in balanced signed base-256 digits
//    F^(b) = sum_a f^(b)_a 256^a, |f| <= 128.
// Then sum_n F[k][n] x_n = sum_a 256^a P_a + K0 R_k (mod p) with the 4 accumulators
// P_a = sum_b sum_n f^(b)_a[k][n] s_{n,b} (|P_a| < 2^22, 16 matrix products per 16 x 16
// tile) and R_k the row sum of F (64 or M2 at k = 0, else 0).  sum_a 256^a P_a < 2^47 is
// formed exactly in float64 and reduced mod p with the exact fp64 remainder of the
// butterfly kernel.
//
// Workgroup: 4 waves, one channel.  Wave w owns block w (16 rows or columns of the
// matrix operand) in every product and holds that block of the matrix digits in registers
// (16 x 16 bytes per lane), the same registers for the 64-point matrix in both forward
// stages (and both inverse stages) when M2 = 64.  Between products the data sit in LDS as
// four digit planes (one per byte) with the next product's contraction index contiguous,
// so that an operand is one 16-byte LDS read; each product is oriented so that the four
// consecutive outputs a lane holds run along that index, and the producer splits its
// results into digits once (a byte transpose) instead of every consumer splitting them.

#include "sc_device.h"
#include "sc_internal.h"

// waves per SIMD the kernel is compiled for (its registers: 512 / waves)
#ifndef SC_NTTM_WAVES
#define SC_NTTM_WAVES 2
#endif

namespace sc {

namespace nttm {

typedef int v4i __attribute__((ext_vector_type(4)));

// 128^{-1} mod p (N^{-1} M2 for N = 128 M2)
constexpr uint64_t ninv_128 = 990445569ull;

constexpr double P = 998244353.0;
constexpr double PINV = 1.0 / 998244353.0;
constexpr double SHIFT = 6755399441055744.0;   // 1.5 * 2^52: x + SHIFT - SHIFT = round(x)
constexpr uint32_t FLIP = 0x00808080u;
// the digits' offset K0 = 0x808080 (below p)
constexpr uint64_t K0P = 0x808080ull;
// LDS digit planes of one 64 x 64 matrix: plane b, row, contraction index k at byte
// b * PLANE + row * 64 + 16 * ((k / 16) ^ ((row / 2) % 4)) + k % 16.  The XOR swizzle of the
// 16-byte chunks puts the 16-byte reads of 8 consecutive rows (one LDS cycle) on 8
// different bank groups.
constexpr int PLANE = 64 * 64;
constexpr int MAT = 4 * PLANE;
__device__ __forceinline__ int at_of(int row, int k)
{
    return row * 64 + (((k >> 4) ^ ((row >> 1) & 3)) << 4) + (k & 15);
}

// a mod p into [-p/2, p/2] (up to one p at the edges), |a| < 2^51
__device__ __forceinline__ double reduce(double a)
{
    const double q = __builtin_fma(a, PINV, SHIFT) - SHIFT;
    return __builtin_fma(-q, P, a);
}
// a * w mod p for a residue word w < p, |a| < 2^36: exact, |result| <= 1.5 p.  The quotient
// estimate uses w / p rounded twice (w * fl(1/p)); it only has to be close for the
// remainder, computed exactly, to stay small.
__device__ __forceinline__ double mulw(double a, uint32_t wu)
{
    const double w = (double)wu;
    const double h = a * w;
    const double l = __builtin_fma(a, w, -h);
    const double q = __builtin_fma(a, w * PINV, SHIFT) - SHIFT;
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
// a residue representative below 2^31 in magnitude as a 32-bit word
__device__ __forceinline__ uint32_t word(double a) { return (uint32_t)(int32_t)a; }

// Four residue words x[0..3] at consecutive contraction indices k0 .. k0 + 3 of one row, into
// the digit planes: plane b gets byte b of each word XOR 0x00808080 (a signed digit).
__device__ __forceinline__ void put4(uint8_t* __restrict__ mat, int row, int k0,
                                     const uint32_t (&x)[4])
{
    const uint32_t w0 = x[0] ^ FLIP, w1 = x[1] ^ FLIP, w2 = x[2] ^ FLIP, w3 = x[3] ^ FLIP;
    // 4 x 4 byte transpose: word b holds byte b of w0..w3
    const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
    const uint32_t t1 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
    const uint32_t t2 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
    const uint32_t t3 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
    uint8_t* at = mat + at_of(row, k0);
    *(uint32_t*)(at) = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    *(uint32_t*)(at + PLANE) = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    *(uint32_t*)(at + 2 * PLANE) = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    *(uint32_t*)(at + 3 * PLANE) = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// the lane's operand: digits of contraction indices 16 g16 .. 16 g16 + 15 of one row, per plane
__device__ __forceinline__ void get16(const uint8_t* __restrict__ mat, int row, int g16,
                                      v4i (&op)[4])
{
    const uint8_t* at = mat + at_of(row, 16 * g16);
#pragma unroll
    for (int b = 0; b < 4; ++b) op[b] = *(const v4i*)(at + b * PLANE);
}

// Matrix digits of block w: F[4 a + b] = lane's 16 bytes of f^(b)_a for rows 16 w + lane%16,
// K = 16 (lane/16) + j (the table is laid out [w][4 a + b][lane][16 bytes]).  The offset is
// made opaque to the compiler, so that each stage's loads stay where they are written
// (hoisted out of the branch loop, the four matrices' digits would all be live at once).
__device__ __forceinline__ void load_digits(const v4i* __restrict__ t, int w, int lane,
                                            v4i (&F)[16])
{
    int z = 0;
    asm volatile("" : "+v"(z));
#pragma unroll
    for (int c = 0; c < 16; ++c) F[c] = t[(w * 16 + c) * 64 + lane + z];
}

// acc[a] = sum_b (matrix digits a, b) x (data digits b): the matrix on the left (LEFT) or
// on the right of the data (the digit matrices are symmetric)
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

// sum_a 256^a acc[a][i] + corr reduced mod p (|result| <= p/2 + 1): the low and high pairs
// in int32 (|acc| < 2^22, so |acc0 + 256 acc1| < 2^31), the rest exact in float64 (< 2^47)
__device__ __forceinline__ double combine(const v4i (&acc)[4], int i, double corr)
{
    const int lo = acc[0][i] + (acc[1][i] << 8);
    const int hi = acc[2][i] + (acc[3][i] << 8);
    return reduce(__builtin_fma((double)hi, 65536.0, (double)lo) + corr);
}

}  // namespace nttm

// Products and layouts (D[row][col] = sum_K Aop[row][K] Bop[K][col]; a lane holds
// D rows 4 (lane/16) + i, i < 4, column lane % 16 of a 16 x 16 tile):
//   S1  D[n2][k1] = sum_{n1} a[n1][n2] F64[n1][k1]   data left,  wave: k1 block
//   S2  D[k2][k1] = sum_{n2} F[k2][n2] B[k1][n2]     data right, wave: k2 block
//   IA  D[k1][m2] = sum_{k2} X[k1][k2] Fi[k2][m2]    data left,  wave: m2 block
//   IB  D[m1][m2] = sum_{k1} Fi64[m1][k1] Z[k1][m2]  data right, wave: m1 block
// and the LDS matrices (row, contiguous contraction index): a as (n2, n1), B as (k1, n2),
// X as (k1, k2), Z as (m2, k1).
template <bool REV>
__global__ __launch_bounds__(256, SC_NTTM_WAVES) void ntt_mfma_kernel(
    const int32_t* __restrict__ v, const int32_t* __restrict__ g, int32_t* __restrict__ r,
    int L, int M2, const nttm::v4i* __restrict__ f64, const nttm::v4i* __restrict__ fm2,
    const nttm::v4i* __restrict__ i64, const nttm::v4i* __restrict__ im2,
    const uint32_t* __restrict__ twf, const uint32_t* __restrict__ twi,
    const uint32_t* __restrict__ tn)
{
    using namespace nttm;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * MAT];
    __shared__ uint32_t vkb[64 * 64];   // V^b at (k1, k2), kept for the product with G^b
    uint8_t* const ma = lds;            // a, then X
    uint8_t* const mb = lds + MAT;      // B, then Z

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int g16 = lane >> 4, c16 = lane & 15;
    const int M = 64 * M2, nb = (M2 + 15) >> 4;   // blocks of 16 holding the M2 dimension
    const int64_t ch = blockIdx.x;
    const Span vs = make_span(v, ch * L, L);
    const Span gs = make_span(g, ch * L, L);
    const Span rs = make_span(r, ch * L, L);
    const double c64 = (double)(K0P * 64ull % 998244353ull);
    const double cm2 = (double)(K0P * (uint64_t)M2 % 998244353ull);
    // the inverse M2-point matrix carries N^{-1}: its column sum at 0 is N^{-1} M2 = 1/128
    const double cmi = (double)(K0P * ninv_128 % 998244353ull);

    v4i F[16], op[4], acc[4];

#pragma unroll 1
    for (int b = 0; b < 2; ++b) {
#pragma unroll 1
        for (int s = 0; s < 2; ++s) {
            // 1. u^b_n = a_n omega_N^{b n}, n = M2 n1 + n2 < M (0 past L), into ma as (n2, n1):
            //    group q = (n2, n1 / 4) holds n1 = 4 (q / M2) + j, n2 = q % M2.  All loads first.
            const Span& src = s == 0 ? vs : gs;
            int32_t raw[4][4];
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int q = tid + 256 * it;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = M2 * (4 * (q / M2) + j) + q % M2;
                    const bool in = q < 16 * M2 && n < L;
                    const int e = (s == 0 && REV) ? L - 1 - n : n;
                    const uint32_t off = in ? (uint32_t)e * 4u : 0x80000000u;
                    raw[it][j] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(src.rs, (int)off,
                                                                              0, 0);
                }
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int q = tid + 256 * it;
                if (q < 16 * M2) {
                    uint32_t x[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int n = M2 * (4 * (q / M2) + j) + q % M2;
                        x[j] = b ? word(mulw((double)raw[it][j], tn[n])) : (uint32_t)raw[it][j];
                    }
                    put4(ma, q % M2, 4 * (q / M2), x);
                }
            }
            // the 64-point matrix for S1 (and S2 when M2 = 64), loaded once the input
            // registers are free
            load_digits(f64, w, lane, F);
            __syncthreads();

            // 2. S1: B = (F64 a) times omega_M^{n2 k1}, into mb as (k1, n2)
#pragma unroll 1
            for (int c = 0; c < nb; ++c) {
                get16(ma, 16 * c + c16, g16, op);
                product<false>(F, op, acc);
                const int k1 = 16 * w + c16;
                uint32_t x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n2 = 16 * c + 4 * g16 + i;
                    const double y = combine(acc, i, k1 == 0 ? c64 : 0.0);
                    x[i] = word(mulw(y, twf[k1 * M2 + (n2 < M2 ? n2 : 0)]));
                }
                put4(mb, k1, 16 * c + 4 * g16, x);
            }
            __syncthreads();

            // 3. S2: A = B F_M2 (A_k at k1, k2 for k = k1 + 64 k2); V kept in LDS, G turned
            //    into X = V G (N^{-1} is folded into the inverse matrix), written to ma as (k1, k2)
            if (M2 < 64) load_digits(fm2, w, lane, F);
            if (16 * w < M2) {
#pragma unroll 1
                for (int rb = 0; rb < 4; ++rb) {
                    get16(mb, 16 * rb + c16, g16, op);
                    product<true>(F, op, acc);
                    const int k1 = 16 * rb + c16;
                    uint32_t x[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int k2 = 16 * w + 4 * g16 + i;
                        const double y = combine(acc, i, k2 == 0 ? cm2 : 0.0);
                        // the same lane reads back what it wrote: no barrier needed
                        if (s == 0)
                            vkb[k1 * 64 + k2] = word(y);
                        else
                            x[i] = word(mulv((double)(int32_t)vkb[k1 * 64 + k2], y));
                    }
                    if (s == 1) put4(ma, k1, 16 * w + 4 * g16, x);
                }
            }
            __syncthreads();
        }

        // 4. IA: Z = X (N^{-1} F_M2^{-1}) times omega_M^{-m2 k1}, into mb as (m2, k1)
        load_digits(im2, w, lane, F);
        if (16 * w < M2) {
#pragma unroll 1
            for (int rb = 0; rb < 4; ++rb) {
                get16(ma, 16 * rb + c16, g16, op);
                product<false>(F, op, acc);
                const int m2 = 16 * w + c16;
                uint32_t x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k1 = 16 * rb + 4 * g16 + i;
                    const double y = combine(acc, i, m2 == 0 ? cmi : 0.0);
                    x[i] = word(mulw(y, twi[k1 * M2 + (m2 < M2 ? m2 : 0)]));
                }
                put4(mb, m2, 16 * rb + 4 * g16, x);
            }
        }
        __syncthreads();

        // 5. IB: e^b = F64^{-1} Z at n = M2 m1 + m2.  Branch 0 parks e^0 in r (the same lane
        //    reads it back); branch 1 forms x_n = e^0_n + omega_N^{-n} e^1_n, lifts and stores it
        load_digits(i64, w, lane, F);
#pragma unroll 1
        for (int c = 0; c < nb; ++c) {
            get16(mb, 16 * c + c16, g16, op);
            product<true>(F, op, acc);
            const int m2 = 16 * c + c16;
            uint32_t prev[4];
            if (b) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = M2 * (16 * w + 4 * g16 + i) + m2;
                    const bool in = m2 < M2 && n < L;
                    const uint32_t off = in ? (uint32_t)(REV ? L - 1 - n : n) * 4u : 0x80000000u;
                    prev[i] = __builtin_amdgcn_raw_buffer_load_b32(rs.rs, (int)off, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m1 = 16 * w + 4 * g16 + i;
                const int n = M2 * m1 + m2;
                const double y = combine(acc, i, m1 == 0 ? c64 : 0.0);
                if (m2 < M2 && n < L) {
                    uint32_t o;
                    if (b == 0) {
                        o = word(y);
                    } else {
                        const double t = mulw(y, tn[(2 * M - n) & (2 * M - 1)]);
                        o = word(balance(reduce(t + (double)(int32_t)prev[i])));
                    }
                    __builtin_amdgcn_raw_buffer_store_b32(o, rs.rs, (REV ? L - 1 - n : n) * 4, 0,
                                                          0);
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
    const nttm::v4i* i64 = (const nttm::v4i*)t.inv64;
    const nttm::v4i* fm2 = (const nttm::v4i*)t.digits[0][lg];
    const nttm::v4i* im2 = (const nttm::v4i*)t.digits[1][lg];
    if (rev)
        hipLaunchKernelGGL((ntt_mfma_kernel<true>), dim3((unsigned)nch), dim3(256), 0, stream, v, g,
                           r, L, M2, f64, fm2, i64, im2, t.twiddle[0][lg], t.twiddle[1][lg],
                           t.roots[lg]);
    else
        hipLaunchKernelGGL((ntt_mfma_kernel<false>), dim3((unsigned)nch), dim3(256), 0, stream, v,
                           g, r, L, M2, f64, fm2, i64, im2, t.twiddle[0][lg], t.twiddle[1][lg],
                           t.roots[lg]);
    return hipGetLastError();
}

}  // namespace sc
