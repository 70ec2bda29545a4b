// Gate stream of the multi-head Fourier module on MFMA (gfx950).
//
// "Caracal: Causal Architecture via Spectral Mixing" (key design 1) makes the convolution
// kernel of each channel from the input: g = Conv1d_G2(sigma(s)) with s a linear projection
// of the normalised activations and Conv1d_G2 a causal convolution with kernel 3 grouped by
// head, so that the channels of one head mix with each other only:
//
//     g[b][co][t] = sum_{i<64} sum_{k<3} W[co][i][k] * sigma(s[b][c0+i][t+k-2])
//
// (c0 the first channel of co's group of 64, the convolution's input zero before t = 0).
// Per token this is a 64 x 192 matrix times a 192-vector, so a tile of T tokens of one group
// is a dense 64 x 192 x T contraction: it runs on the matrix cores, as three shifted
// products W_k (64 x 64) * sigma(S)[:, t+k-2] accumulated in fp32.
//
// One workgroup (4 waves) per (batch row, group, tile of T tokens):
//  1. sigma(s) for tokens t0-2 .. t0+T-1 into LDS, one row per token (the 64 channels of
//     the group contiguous), zero before t = 0; bf16 storage rounds sigma to bf16, the
//     precision a bf16 layer computes it in.
//  2. the group's W (64 x 64 x 3, contiguous) is read with 16-byte loads and passed through
//     LDS (before the sigma tile, in the same space) into registers: each wave holds the W
//     fragments of its 32 output channels (all 3 taps, all 64 inputs) and accumulates
//     32 x 32 output blocks over T/2 tokens;
//  3. the blocks go through LDS to coalesced stores of g rows (channel-major, t contiguous).
// s is read token-major ((B, L, C): one 64-channel row per token, 16-byte vector loads) or
// channel-major ((B, C, L): t contiguous). Channel-major bf16 rows whose length is a multiple
// of 8 and that start 16-byte aligned are read with 16-byte vectors along t into a
// channel-row LDS tile and turned into token rows by an LDS transpose (sigma applied on the
// way); other channel-major shapes use element loads.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "sc_device.h"
#include "sc_internal.h"

namespace sc {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

constexpr int GT = 256;      // threads
// waves per SIMD the token-major bf16 form is compiled for (registers <= 512 / waves; the
// fp32 form takes 3, which its 50 KB of LDS allows anyway)
#ifndef SC_GATE_TM_WAVES
#define SC_GATE_TM_WAVES 5
#endif
constexpr int GC = 64;       // channels per group

template <class IO>
struct GateCfg;

template <>
struct GateCfg<bf16_io> {
    static constexpr int T = 128;       // tokens per tile
    static constexpr int SP = 72;       // LDS row pitch (elements): 144 bytes
    static constexpr int KS = 16;       // reduction depth of one MFMA
};

template <>
struct GateCfg<f32_io> {
    static constexpr int T = 128;
    static constexpr int SP = 65;
    static constexpr int KS = 2;
};

// 1 / (1 + e^-x) with the hardware exponential and reciprocal (each about 1 ulp; far below
// the fp32 tolerance of this path and below the rounding of sigma to bf16)
__device__ __forceinline__ float sigmoid(float x)
{
    return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

__device__ __forceinline__ uint16_t to_bf16(float x) { return (uint16_t)pack_bf16x2(x, 0.f); }

template <class IO, bool TM, bool VIN>
__global__ __launch_bounds__(GT, VIN ? 4 : (TM ? (sizeof(typename IO::T) == 2 ? SC_GATE_TM_WAVES : 3) : 1)) void gate_kernel(const typename IO::T* __restrict__ s,
                                                  const typename IO::T* __restrict__ W,
                                                  typename IO::T* __restrict__ g, int C, int L,
                                                  int gcs, int ngroups, int ntiles, int vec_out)
{
    using E = typename IO::T;
    constexpr bool BF = sizeof(E) == 2;
    constexpr int T = GateCfg<IO>::T, SP = GateCfg<IO>::SP, KS = GateCfg<IO>::KS;
    constexpr int CS = GC / KS;          // MFMA steps per tap
    constexpr int NB = T / 64;           // 32-token blocks per wave
    constexpr int S_BYTES = (T + 2) * SP * (int)sizeof(E);
    constexpr int O_BYTES = GC * T * (int)sizeof(E);
    // W rows of one output channel (192 elements) padded so that the 32 lanes of a fragment
    // read (32 output channels) spread over the LDS banks, and 16-byte aligned
    constexpr int WP = GC * 3 + (BF ? 8 : 4);
    constexpr int W_BYTES = GC * WP * (int)sizeof(E);
    // VIN: channel rows of the tile, N[ci][NP]: tokens t0 .. t0+T-1, then t0-2 and t0-1,
    // padded so that each row starts 16-byte aligned; right after S, in space W has used
    // (N is written once every wave holds its W fragments, and read while S is written):
    // 36 KB of LDS and at most 128 registers keep four workgroups on a CU
    static_assert(!VIN || (BF && !TM), "vector channel-major input is a bf16 path");
    constexpr int NP = T + 8;
    constexpr int NOFF = S_BYTES;
    static_assert(!VIN || (NOFF % 16 == 0 && (NP * (int)sizeof(E)) % 16 == 0), "16-byte rows");
    constexpr int SN_BYTES = VIN ? NOFF + GC * NP * (int)sizeof(E) : S_BYTES;
    constexpr int SO_BYTES = SN_BYTES > O_BYTES ? SN_BYTES : O_BYTES;
    constexpr int LDS_BYTES = SO_BYTES > W_BYTES ? SO_BYTES : W_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
    E* S = (E*)smem;                     // S[tt][ci], tt = t - t0 + 2
    E* O = (E*)smem;                     // O[co][tl], after the products
    E* Wl = (E*)smem;                    // Wl[co * WP + ci * 3 + k], before the sigma tile
    E* N = (E*)(smem + NOFF);            // VIN only

    uint32_t id = blockIdx.x;
    const int tile = (int)(id % (uint32_t)ntiles);
    id /= (uint32_t)ntiles;
    const int grp = (int)(id % (uint32_t)ngroups);
    const int64_t z = id / (uint32_t)ngroups;
    const int t0 = tile * T, c0 = grp * GC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // all global loads first: the group's W (64 * 192 contiguous elements, 16-byte vectors,
    // W 16-byte aligned) and this tile's s, then W through LDS into registers, then sigma(s)
    // into the same LDS space
    constexpr int WEPV = 16 / (int)sizeof(E), WNV = GC * GC * 3 / WEPV / GT;
    uint4 wraw[WNV];
    const E* wg = W + (int64_t)c0 * (GC * 3);
#pragma unroll
    for (int q = 0; q < WNV; ++q) wraw[q] = *(const uint4*)(wg + (tid + GT * q) * WEPV);

    constexpr int EPV = 16 / (int)sizeof(E);          // elements per 16-byte vector
    constexpr int VPR = GC / EPV;                     // vectors per token row (token-major)
    constexpr int NV = T * VPR / GT;                  // token-major vectors per thread
    constexpr int NE = T * GC / GT;                   // channel-major elements per thread
    constexpr int VPC = T / EPV;                      // vectors per channel row (VIN)
    constexpr int NVC = GC * VPC / GT;                // VIN vectors per thread
    uint4 raw[TM ? NV : 1];
    // VIN: the tile's 16-byte vectors as one vector value (held across the W fragment reads;
    // an array there was kept in scratch memory)
    static_assert(!VIN || NVC == 4, "four vectors per thread");
    u32x16 rv = {};
    float val[(TM || VIN) ? 1 : NE];
    uint4 halo = make_uint4(0, 0, 0, 0);
    float hv = 0.f;
    uint32_t hw = 0;
    const int hr = TM ? tid / VPR : (tid & 1);
    const int hc = TM ? tid % VPR : (tid >> 1);
    const int ht = t0 - 2 + hr;
    const bool hact = tid < (TM ? 2 * VPR : 2 * GC) && ht >= 0;
    if constexpr (TM) {
        const E* sz = s + z * (int64_t)L * C + c0;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int vid = tid + GT * q, r = vid / VPR, p = vid % VPR;
            const int tc = t0 + r < L ? t0 + r : L - 1;
            raw[q] = *(const uint4*)(sz + (int64_t)tc * C + p * EPV);
        }
        if (hact) halo = *(const uint4*)(sz + (int64_t)ht * C + hc * EPV);
    } else if constexpr (VIN) {
        // L is a multiple of 8 and rows are 16-byte aligned: a vector lies wholly inside or
        // wholly past the row (then it is clamped to the last one and later zeroed); the halo
        // tokens t0-2, t0-1 of channel tid are one aligned 4-byte word, present when t0 > 0
        const E* sz = s + (z * C + c0) * (int64_t)L;
#pragma unroll
        for (int q = 0; q < NVC; ++q) {
            const int vid = tid + GT * q, ci = vid / VPC, p = vid % VPC;
            const int tv = t0 + p * EPV < L ? t0 + p * EPV : L - EPV;
            const uint4 w = *(const uint4*)(sz + (int64_t)ci * L + tv);
            rv[4 * q] = w.x;
            rv[4 * q + 1] = w.y;
            rv[4 * q + 2] = w.z;
            rv[4 * q + 3] = w.w;
        }
        if (tid < GC && t0 > 0) hw = *(const uint32_t*)(sz + (int64_t)tid * L + t0 - 2);
    } else {
        const E* sz = s + (z * C + c0) * (int64_t)L;
#pragma unroll
        for (int q = 0; q < NE; ++q) {
            const int e = tid + GT * q, r = e % T, ci = e / T;
            const int tc = t0 + r < L ? t0 + r : L - 1;
            val[q] = IO::load(sz, (int64_t)ci * L + tc);
        }
        if (hact) hv = IO::load(sz, (int64_t)hc * L + ht);
    }

    // W into LDS, row by row (a 16-byte vector never crosses a 192-element row)
#pragma unroll
    for (int q = 0; q < WNV; ++q) {
        const int f = (tid + GT * q) * WEPV;
        *(uint4*)(Wl + (f / (GC * 3)) * WP + f % (GC * 3)) = wraw[q];
    }
    __syncthreads();

    // 2. this wave's W fragments: A[i = co][kk = ci] of tap k
    const int cb = wave & 1, th = wave >> 1;
    const int col = 32 * cb + (lane & 31);
    const int half = lane >> 5;
    f32x16 acc[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
    using AF = typename std::conditional<BF, uint4, float>::type;
    AF a[3][CS];
    const E* wl = Wl + col * WP + (BF ? 8 * half : half) * 3;   // then + (KS cs + e) 3 + k
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) {
            if constexpr (BF) {
                uint32_t u[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    u[e] = (uint32_t)wl[(KS * cs + 2 * e) * 3 + k] |
                           ((uint32_t)wl[(KS * cs + 2 * e + 1) * 3 + k] << 16);
                a[k][cs] = make_uint4(u[0], u[1], u[2], u[3]);
            } else {
                a[k][cs] = wl[KS * cs * 3 + k];
            }
        }
    __syncthreads();   // every wave has its fragments: the space takes sigma(s) now

    // 1 (cont.). sigma(s) into LDS: S[tt][ci], zero before t = 0 and from t = L on
    if constexpr (TM) {
        auto put = [&](int row, int cc, const uint4& w, bool valid) {
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
            if constexpr (BF) {
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = valid ? sigmoid(__uint_as_float(u[e] << 16)) : 0.f;
                    const float hi = valid ? sigmoid(__uint_as_float(u[e] & 0xffff0000u)) : 0.f;
                    o[e] = pack_bf16x2(lo, hi);
                }
                *(uint4*)(S + row * SP + cc) = make_uint4(o[0], o[1], o[2], o[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[row * SP + cc + e] = valid ? sigmoid(__uint_as_float(u[e])) : 0.f;
            }
        };
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int vid = tid + GT * q, r = vid / VPR, p = vid % VPR;
            put(r + 2, p * EPV, raw[q], t0 + r < L);
        }
        if (tid < 2 * VPR) put(hr, hc * EPV, halo, ht >= 0);
    } else if constexpr (VIN) {
        // the tile's channel rows into N, then
#pragma unroll
        for (int q = 0; q < NVC; ++q) {
            const int vid = tid + GT * q, ci = vid / VPC, p = vid % VPC;
            *(uint4*)(N + ci * NP + p * EPV) = make_uint4(rv[4 * q], rv[4 * q + 1], rv[4 * q + 2], rv[4 * q + 3]);
        }
        if (tid < GC) *(uint32_t*)(N + tid * NP + T) = hw;
        __syncthreads();
        // transpose: 8 channels of one token column into one 16-byte token-row vector;
        // consecutive lanes take consecutive tokens (conflict-free 2-byte reads)
        auto row8 = [&](int col, int cg, bool valid) {
            const E* nc = N + 8 * cg * NP + col;
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = valid ? sigmoid(__uint_as_float((uint32_t)nc[2 * e * NP] << 16)) : 0.f;
                const float hi = valid ? sigmoid(__uint_as_float((uint32_t)nc[(2 * e + 1) * NP] << 16)) : 0.f;
                o[e] = pack_bf16x2(lo, hi);
            }
            return make_uint4(o[0], o[1], o[2], o[3]);
        };
        static_assert(T * (GC / 8) % GT == 0, "whole transpose rounds");
#pragma unroll
        for (int q = 0; q < T * (GC / 8) / GT; ++q) {
            const int vid = tid + GT * q, j = vid % T, cg = vid / T;
            *(uint4*)(S + (j + 2) * SP + 8 * cg) = row8(j, cg, t0 + j < L);
        }
        if (tid < 2 * (GC / 8)) {
            const int r = tid / (GC / 8), cg = tid % (GC / 8);
            *(uint4*)(S + r * SP + 8 * cg) = row8(T + r, cg, t0 > 0);
        }
    } else {
#pragma unroll
        for (int q = 0; q < NE; ++q) {
            const int e = tid + GT * q, r = e % T, ci = e / T;
            const float x = t0 + r < L ? sigmoid(val[q]) : 0.f;
            if constexpr (BF) S[(r + 2) * SP + ci] = to_bf16(x);
            else S[(r + 2) * SP + ci] = x;
        }
        if (tid < 2 * GC) {
            const float x = ht >= 0 ? sigmoid(hv) : 0.f;
            if constexpr (BF) S[hr * SP + hc] = to_bf16(x);
            else S[hr * SP + hc] = x;
        }
    }
    __syncthreads();

    // 2 (cont.). the products
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int cs = 0; cs < CS; ++cs)
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                const int tl = th * (T / 2) + 32 * m + (lane & 31);
                if constexpr (BF) {
                    const uint4 bw = *(const uint4*)(S + (tl + k) * SP + KS * cs + 8 * half);
                    acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a[k][cs]), __builtin_bit_cast(bf16x8, bw),
                        acc[m], 0, 0, 0);
                } else {
                    const float bv = S[(tl + k) * SP + KS * cs + half];
                    acc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[k][cs], bv, acc[m], 0, 0, 0);
                }
            }
    __syncthreads();   // every wave is done reading S

    // 3. blocks to LDS (output storage type), then whole rows to g
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        const int tl = th * (T / 2) + 32 * m + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r >> 2) + 4 * half + (r & 3);
            if constexpr (BF) O[(32 * cb + i) * T + tl] = to_bf16(acc[m][r]);
            else O[(32 * cb + i) * T + tl] = acc[m][r];
        }
    }
    __syncthreads();
    E* gz = g + (z * gcs + c0) * (int64_t)L;
    if (vec_out) {
        // L is a multiple of the vector's elements and g rows are 16-byte aligned
        constexpr int OVPR = T / EPV, ONV = GC * OVPR / GT;
#pragma unroll
        for (int q = 0; q < ONV; ++q) {
            const int vid = tid + GT * q, row = vid / OVPR, p = vid % OVPR;
            if (t0 + p * EPV < L)
                *(uint4*)(gz + (int64_t)row * L + t0 + p * EPV) = *(const uint4*)(O + row * T + p * EPV);
        }
    } else {
        constexpr int ONE = GC * T / GT;
#pragma unroll
        for (int q = 0; q < ONE; ++q) {
            const int e = tid + GT * q, tl = e % T, row = e / T;
            if (t0 + tl < L) gz[(int64_t)row * L + t0 + tl] = O[row * T + tl];
        }
    }
}

template <class IO, bool TM, bool VIN = false>
hipError_t gate_launch(const void* s, const void* W, void* g, int64_t nb, int64_t C, int64_t cw,
                       int64_t L, int64_t gcs, bool vec_out, hipStream_t st)
{
    constexpr int T = GateCfg<IO>::T;
    const int64_t ntiles = (L + T - 1) / T, ngroups = cw / GC;
    const int64_t blocks = ntiles * ngroups * nb;
    if (blocks <= 0) return hipSuccess;
    if (!grid_ok(blocks, GT)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gate_kernel<IO, TM, VIN>), dim3((unsigned)blocks), dim3(GT), 0, st,
                       (const typename IO::T*)s, (const typename IO::T*)W, (typename IO::T*)g,
                       (int)C, (int)L, (int)gcs, (int)ngroups, (int)ntiles, vec_out ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate(Store st, bool token_major, const void* s, const void* W, void* g,
                       int64_t nb, int64_t C, int64_t cw, int64_t L, int64_t gcs, hipStream_t s_)
{
    const size_t es = st == Store::F32 ? 4 : 2;
    const bool vec_out = L % (int64_t)(16 / es) == 0 && (uintptr_t)g % 16 == 0;
    if (st == Store::F32)
        return token_major ? gate_launch<f32_io, true>(s, W, g, nb, C, cw, L, gcs, vec_out, s_)
                           : gate_launch<f32_io, false>(s, W, g, nb, C, cw, L, gcs, vec_out, s_);
    if (token_major) return gate_launch<bf16_io, true>(s, W, g, nb, C, cw, L, gcs, vec_out, s_);
    // channel-major bf16 rows: 16-byte input vectors when every row starts aligned
    const bool vec_in = L % 8 == 0 && (uintptr_t)s % 16 == 0;
    return vec_in ? gate_launch<bf16_io, false, true>(s, W, g, nb, C, cw, L, gcs, vec_out, s_)
                  : gate_launch<bf16_io, false>(s, W, g, nb, C, cw, L, gcs, vec_out, s_);
}

}  // namespace sc
