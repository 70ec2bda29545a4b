// Internal (non-exported) interface between the host ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sc {

// Length of the shared float twiddle table used by the fused path: tw[i] = W_8192^i.
constexpr int FUSED_TW_N = 8192;
// The float twiddle bank: W_8192^i (i < 8192); then for each radix-16 pass length
// Q = 32..4096 a table of W_Q^{n k} stored row k (k < 16), column n (n < Q/16); then for
// each radix-8 pass length Q = 16..4096 the same with k < 8, n < Q/8.  Q entries per Q.
constexpr int FUSED_BANK_FLOAT2 = FUSED_TW_N + (4096 * 2 - 32) + (4096 * 2 - 16);
// Largest sequence length handled by the one-workgroup-per-channel (fused) kernels.
constexpr int FUSED_MAX_L = 4096;
// Sequences up to this length are computed entirely by direct summation.
constexpr int DIRECT_MAX_L = 32;

enum class Store { F32, BF16 };

// Every launcher computes r = causal(v, g) per channel; with rev it computes the gradient
// form r = rev(causal(rev(v), g)), i.e. r_j = sum_{t>=j} v_t g_{t-j} (v read reversed, r
// written reversed).

// Fused in-LDS causal convolution for DIRECT_MAX_L < L <= FUSED_MAX_L.
// M = next power of two >= L.  head = number of leading outputs computed directly (even).
hipError_t launch_fused(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                        int M, int head, bool pair_store, bool rev, const float2* tw,
                        hipStream_t stream);

// Constants of the exact path modulo p = 998244353 (omega_n = 3^((p-1)/n)).  The bank
// holds pairs of doubles {w, w / p}:
//   [0, 8192)                               w = omega_8192^i
//   [NTT_PASS_BASE + (Q - 32) + k*(Q/16) + n] w = omega_Q^{n k}, Q = 32 .. 4096, k < 16, n < Q/16
// ninv[k] = (2^k)^{-1} mod p as a double, ninv_q[k] = ninv[k] / p.
constexpr int NTT_TW_N = 8192;
constexpr int NTT_PASS_BASE = NTT_TW_N;
constexpr int NTT_BANK_ENTRIES = NTT_TW_N + (2 * 4096 - 32);
struct NttTables {
    const double* bank = nullptr;
    double ninv[24];
    double ninv_q[24];
};

// The exact paths' primes: A = 998244353 (the exact int32 kind), B = 1004535809 and
// C = 469762049; all have 2^21 | p - 1 and primitive root 3.
constexpr uint64_t NTT_PRIMES[3] = {998244353ull, 1004535809ull, 469762049ull};

// Exact NTT causal convolution for L <= FUSED_MAX_L, M = max(64, next power of two >= L),
// modulo prime A, output lifted to the balanced range.
hipError_t launch_ntt(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch, int L, int M,
                      bool rev, const NttTables& tables, hipStream_t stream);

// Exact real-valued causal convolution: V = round(v 2^fv), G = round(g 2^fg), the exact
// integer sum R through primes A, B, C (tables[0..2]) into scratch (3 * nch * L int32), then
// r = round_f32(R 2^-(fv+fg)).
hipError_t launch_fixed(const float* v, const float* g, float* r, int32_t* scratch, int64_t nch,
                        int L, int M, int fv, int fg, const NttTables* tables, hipStream_t stream);

// ---- four-step path (L > FUSED_MAX_L)
// Longest row transform of the four-step split M = M1 * M2 (M2 <= this, M1 >= 64).
constexpr int FOURSTEP_MAX_ROW = 4096;
// Largest sequence length of the four-step path (N = 2M <= 2^23 divides p - 1 as well).
constexpr int64_t FOURSTEP_MAX_L = (int64_t)1 << 22;

// Twiddle tables of the four-step path for one M = M1 * M2 (N = 2M, H = M2/2):
//   tn[e]                          W_N^e, e < N
//   ta[k2 * M2 + n1]               W_M^{n1 k2}        (k2 < M1, n1 < M2)
//   tb[i2 * H + m1]                W_{M/2}^{m1 i2}    (i2 < M1, m1 < H)
//   tu[(2 rho + b) * (M2/4 + 1) + k1]  W_N^{2 (M1 k1 + rho) + b}   (rho < M1, b < 2, k1 <= M2/4)
struct FsTw {
    const float2* tn;
    const float2* ta;
    const float2* tb;
    const float2* tu;
};

// A 1-D launch keeps its block count below 2^31 and its work-items below 2^32 (the dispatch
// packet's grid size is 32 bits); launchers refuse larger grids with hipErrorInvalidValue.
inline bool grid_ok(int64_t blocks, int64_t threads)
{
    return blocks >= 0 && blocks <= 0x7fffffff && blocks * threads <= 0xffffffffLL;
}

void fourstep_split(int M, int* M1, int* M2);
size_t fourstep_bytes_per_channel(int M);
// ws holds chunk channels of scratch (chunk * fourstep_bytes_per_channel(M) bytes).  With a
// second stream `side` (and two events, fork and join), the channels go in parts of chunk/2
// that alternate between the two streams, each part with its own half of ws: side waits
// for stream at the start (fork) and stream for side at the end (join), so the call stays
// ordered on `stream` as a whole.
hipError_t launch_fourstep(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                           int M, int head, bool pair_store, bool rev, const float2* bank,
                           const FsTw& tw, void* ws, int64_t chunk, hipStream_t stream,
                           hipStream_t side, hipEvent_t fork, hipEvent_t join);

// ---- filter shared by the batch (L <= FUSED_MAX_L, M = max(64, next power of two >= L))
// Spectrum of the filters k[C][L]: shared_spec_stride(M) float2 per channel.
int64_t shared_spec_stride(int M);
hipError_t launch_shared_spectrum(Store st, const void* k, float2* spec, int C, int L, int M,
                                  const float2* tw, hipStream_t stream);
// r[b][c][t] = sum_{j<=t} v[b][c][j] k[c][t-j] from the spectrum; B * C * L elements of v and
// r must stay below 2^31 bytes (the host splits larger batches).
// With rev: r[b][c][j] = sum_{t>=j} v[b][c][t] k[c][t-j] (the gradient dv for v = dr).
hipError_t launch_shared_apply(Store st, const void* v, const float2* spec, void* r, int B, int C,
                               int L, int M, int head, bool rev, const float2* tw,
                               hipStream_t stream);
// dk[c][j] = sum_b sum_{t>=j} dr[b][c][t] v[b][c][t-j]; pair_store as the fused kernel's.
hipError_t launch_shared_dk(Store st, const void* dr, const void* v, void* dk, int B, int C, int L,
                            int M, int head, bool pair_store, const float2* tw, hipStream_t stream);
// workgroups launch_shared_bwd uses for C channels at transform length M
int64_t shared_bwd_blocks(int64_t C, int M);
// gradients for the upstream gradient dr: dv[b][c][j] = sum_{t>=j} dr[b][c][t] k[c][t-j] from
// the spectrum, dk[c][j] = sum_b sum_{t>=j} dr[b][c][t] v[b][c][t-j]; pair_store as the fused
// kernel's (for both outputs).  C L elements stay below 2^31 bytes (host check).
hipError_t launch_shared_bwd(Store st, const void* dr, const void* v, const float2* spec, void* dv,
                             void* dk, int B, int C, int L, int M, int head, bool pair_store,
                             const float2* tw, hipStream_t stream);
// dk of an empty batch (the sum over no rows): n16 halfwords of p set to zero by a kernel
// (no memset node, so the call can be captured into a graph)
hipError_t launch_zero16(void* p, int64_t n16, hipStream_t stream);

// Direct summation r_t = sum_{j<=t} v_j g_{t-j} in fp32, one thread per output.
hipError_t launch_direct(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                         bool rev, hipStream_t stream);

// dst[z dz + j ds + i] = src[z sz + i ss + j] for i < R, j < Cc, z < nz, of 2- or 4-byte
// elements, for the pair (src0, dst0) and, when src1 is not null, (src1, dst1); dst_major
// orders the tiles along the destination rows (for a destination in HBM), else along the
// source rows
hipError_t launch_transpose(int elt_bytes, const void* src0, void* dst0, const void* src1,
                            void* dst1, int64_t R, int64_t Cc, int64_t ss, int64_t ds, int64_t sz,
                            int64_t dz, int64_t nz, bool dst_major, hipStream_t s);

// g = Conv1d_G2(sigma(s)) for nb batch rows and the cw channels (whole groups of 64) of a
// chunk: s token-major (element (z, c, t) at z L C + t C + c, 16-byte aligned) or
// channel-major (at (z C + c) L + t) with C the channel count of s's rows; W (cw, 64, 3) of
// the chunk; g channel-major with gcs channels per batch row
hipError_t launch_gate(Store st, bool token_major, const void* s, const void* W, void* g,
                       int64_t nb, int64_t C, int64_t cw, int64_t L, int64_t gcs, hipStream_t s_);

}  // namespace sc
