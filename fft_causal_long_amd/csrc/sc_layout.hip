// Layout change between the token-major (B, L, C) tensors of a model layer and the
// channel-major rows the convolution kernels read (gfx950).
//
// The Caracal notes build v and g by linear projections of the normalised activations
// ("Caracal: Causal Architecture via Spectral Mixing", key design 1), so in a model they
// arrive token-major: element (b, t, c) at (b L + t) C + c.  A convolution workgroup needs
// one channel's whole sequence; read in place, every 128-byte line of a (B, L, C) tensor
// carries 32 to 64 channels of one position, so each workgroup would pull a line through
// L2 for each 2 or 4 useful bytes.  The library instead moves a chunk of channels at a
// time between the two layouts with this tiled transpose (both sides coalesced) into a
// workspace small enough to stay in the 256 MB last-level cache, and runs the ordinary
// kernels on the workspace.
//
// transpose_kernel: for each of npair (src, dst) pairs and each batch z < nz,
//     dst[z dz + j ds + i] = src[z sz + i ss + j],   i < R, j < Cc
// in 64 x 64 tiles through LDS; one workgroup per tile, the tiles of all pairs and batches
// in one flat grid.  Elements are moved as raw 2- or 4-byte words.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sc_internal.h"

namespace sc {

namespace {

constexpr int TT = 64;          // tile edge
constexpr int TP_THREADS = 256;

template <typename W>
__global__ __launch_bounds__(TP_THREADS) void transpose_kernel(
    const W* __restrict__ src0, W* __restrict__ dst0, const W* __restrict__ src1,
    W* __restrict__ dst1, int64_t R, int64_t Cc, int64_t ss, int64_t ds, int64_t sz, int64_t dz,
    int64_t nz, int64_t tr, int64_t tc, int dst_major)
{
    __shared__ uint32_t tile[TT][TT + 1];
    // consecutive workgroups take neighbouring tiles along the source rows, or with
    // dst_major along the destination rows, so that the side in HBM is visited in order
    // (the grid has fewer than 2^31 tiles, so the decomposition runs in 32 bits)
    uint32_t id = blockIdx.x, it, jt;
    if (dst_major) {
        it = id % (uint32_t)tr;
        id /= (uint32_t)tr;
        jt = id % (uint32_t)tc;
        id /= (uint32_t)tc;
    } else {
        jt = id % (uint32_t)tc;
        id /= (uint32_t)tc;
        it = id % (uint32_t)tr;
        id /= (uint32_t)tr;
    }
    const int64_t z = id % (uint32_t)nz;
    const int pair = (int)(id / (uint32_t)nz);
    const W* src = (pair ? src1 : src0) + z * sz;
    W* dst = (pair ? dst1 : dst0) + z * dz;
    const int64_t i0 = (int64_t)it * TT, j0 = (int64_t)jt * TT;
    const int tx = threadIdx.x % TT, ty = threadIdx.x / TT;

    // rows i0 + ty + 4k of the source, columns j0 + tx: one coalesced row per wave.  Indices
    // past the matrix are clamped to its last row / column, so every load is unconditional
    // and all of them are in flight together; those values are never stored.
    const int64_t jc = j0 + tx < Cc ? j0 + tx : Cc - 1;
    uint32_t w[TT / 4];
#pragma unroll
    for (int k = 0; k < TT / 4; ++k) {
        const int64_t ic = i0 + ty + 4 * k < R ? i0 + ty + 4 * k : R - 1;
        w[k] = (uint32_t)src[ic * ss + jc];
    }
#pragma unroll
    for (int k = 0; k < TT / 4; ++k) tile[ty + 4 * k][tx] = w[k];
    __syncthreads();
    // rows j0 + ty + 4k of the destination, columns i0 + tx
    const bool iin = i0 + tx < R;
#pragma unroll
    for (int k = 0; k < TT / 4; ++k) {
        const int jj = ty + 4 * k;
        if (iin && j0 + jj < Cc) dst[(j0 + jj) * ds + i0 + tx] = (W)tile[tx][jj];
    }
}

// The same with element pairs: each lane loads columns (j, j+1) of a source row as one
// word and stores rows (i, i+1) of a destination row as one word (4 bytes for 2-byte
// elements, 8 for 4-byte ones), so a wave moves two 64-element rows per instruction.  Needs
// even R, Cc, strides and element offsets (the host checks).
template <typename E, typename P>
__global__ __launch_bounds__(TP_THREADS) void transpose_pair_kernel(
    const E* __restrict__ src0, E* __restrict__ dst0, const E* __restrict__ src1,
    E* __restrict__ dst1, int64_t R, int64_t Cc, int64_t ss, int64_t ds, int64_t sz, int64_t dz,
    int64_t nz, int64_t tr, int64_t tc, int dst_major)
{
    __shared__ E tile[TT][TT + (sizeof(E) == 4 ? 1 : 2)];
    // consecutive workgroups take neighbouring tiles along the source rows, or with
    // dst_major along the destination rows, so that the side in HBM is visited in order
    // (the grid has fewer than 2^31 tiles, so the decomposition runs in 32 bits)
    uint32_t id = blockIdx.x, it, jt;
    if (dst_major) {
        it = id % (uint32_t)tr;
        id /= (uint32_t)tr;
        jt = id % (uint32_t)tc;
        id /= (uint32_t)tc;
    } else {
        jt = id % (uint32_t)tc;
        id /= (uint32_t)tc;
        it = id % (uint32_t)tr;
        id /= (uint32_t)tr;
    }
    const int64_t z = id % (uint32_t)nz;
    const int pair = (int)(id / (uint32_t)nz);
    const E* src = (pair ? src1 : src0) + z * sz;
    E* dst = (pair ? dst1 : dst0) + z * dz;
    const int64_t i0 = (int64_t)it * TT, j0 = (int64_t)jt * TT;
    const int hx = threadIdx.x % (TT / 2), hy = threadIdx.x / (TT / 2);   // 32 x 8

    // clamped, unconditional loads as in transpose_kernel (Cc is even, so Cc - 2 starts a pair)
    const int64_t jc = j0 + 2 * hx < Cc ? j0 + 2 * hx : Cc - 2;
    P w[TT / 8];
#pragma unroll
    for (int k = 0; k < TT / 8; ++k) {
        const int64_t ic = i0 + hy + 8 * k < R ? i0 + hy + 8 * k : R - 1;
        w[k] = *(const P*)(src + ic * ss + jc);
    }
#pragma unroll
    for (int k = 0; k < TT / 8; ++k) {
        const E* e = (const E*)&w[k];
        tile[hy + 8 * k][2 * hx] = e[0];
        tile[hy + 8 * k][2 * hx + 1] = e[1];
    }
    __syncthreads();
    const bool iin = i0 + 2 * hx < R;
#pragma unroll
    for (int k = 0; k < TT / 8; ++k) {
        const int jj = hy + 8 * k;
        if (iin && j0 + jj < Cc) {
            P w;
            E* e = (E*)&w;
            e[0] = tile[2 * hx][jj];
            e[1] = tile[2 * hx + 1][jj];
            *(P*)(dst + (j0 + jj) * ds + i0 + 2 * hx) = w;
        }
    }
}

}  // namespace

hipError_t launch_transpose(int elt_bytes, const void* src0, void* dst0, const void* src1,
                            void* dst1, int64_t R, int64_t Cc, int64_t ss, int64_t ds, int64_t sz,
                            int64_t dz, int64_t nz, bool dst_major, hipStream_t s)
{
    if (R <= 0 || Cc <= 0 || nz <= 0) return hipSuccess;
    const int64_t tr = (R + TT - 1) / TT, tc = (Cc + TT - 1) / TT;
    const int64_t blocks = tr * tc * nz * (src1 ? 2 : 1);
    if (!grid_ok(blocks, TP_THREADS)) return hipErrorInvalidValue;
    const bool even = ((R | Cc | ss | ds | sz | dz) & 1) == 0 &&
                      ((uintptr_t)src0 | (uintptr_t)dst0 | (uintptr_t)src1 | (uintptr_t)dst1) %
                              (2 * elt_bytes) == 0;
    if (even && elt_bytes == 2) {
        hipLaunchKernelGGL((transpose_pair_kernel<uint16_t, uint32_t>), dim3((unsigned)blocks),
                           dim3(TP_THREADS), 0, s, (const uint16_t*)src0, (uint16_t*)dst0,
                           (const uint16_t*)src1, (uint16_t*)dst1, R, Cc, ss, ds, sz, dz, nz, tr,
                           tc, dst_major ? 1 : 0);
        return hipGetLastError();
    }
    if (even && elt_bytes == 4) {
        hipLaunchKernelGGL((transpose_pair_kernel<uint32_t, uint2>), dim3((unsigned)blocks),
                           dim3(TP_THREADS), 0, s, (const uint32_t*)src0, (uint32_t*)dst0,
                           (const uint32_t*)src1, (uint32_t*)dst1, R, Cc, ss, ds, sz, dz, nz, tr,
                           tc, dst_major ? 1 : 0);
        return hipGetLastError();
    }
    if (elt_bytes == 2)
        hipLaunchKernelGGL(transpose_kernel<uint16_t>, dim3((unsigned)blocks), dim3(TP_THREADS), 0,
                           s, (const uint16_t*)src0, (uint16_t*)dst0, (const uint16_t*)src1,
                           (uint16_t*)dst1, R, Cc, ss, ds, sz, dz, nz, tr, tc,
                           dst_major ? 1 : 0);
    else if (elt_bytes == 4)
        hipLaunchKernelGGL(transpose_kernel<uint32_t>, dim3((unsigned)blocks), dim3(TP_THREADS), 0,
                           s, (const uint32_t*)src0, (uint32_t*)dst0, (const uint32_t*)src1,
                           (uint32_t*)dst1, R, Cc, ss, ds, sz, dz, nz, tr, tc,
                           dst_major ? 1 : 0);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace sc
