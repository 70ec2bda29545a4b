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

// Workgroups of `kernel` (threads per workgroup, static LDS only) resident at once on the
// current device: the occupancy calculator's workgroups per CU times the CU count, cached per
// device in `cache` (0: not known yet).  0 if a query fails (its error is cleared).
inline int64_t resident_workgroups(const void* kernel, int threads, int64_t (&cache)[16])
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) {
        (void)hipGetLastError();
        return 0;
    }
    const int64_t known = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (known > 0) return known;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    const int64_t n = (int64_t)cus * per_cu;
    __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
    return n;
}

// Every launcher computes r = causal(v, g) per channel; with rev it computes the gradient
// form r = rev(causal(rev(v), g)), i.e. r_j = sum_{t>=j} v_t g_{t-j} (v read reversed, r
// written reversed).

// Fused in-LDS causal convolution for DIRECT_MAX_L < L <= FUSED_MAX_L.
// M = next power of two >= L.  head = number of leading outputs computed directly (even).
hipError_t launch_fused(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                        int M, int head, bool pair_store, bool rev, const float2* tw,
                        hipStream_t stream);

// The M = 4096 fused kernel (sc_fused4k.hip): its twiddle table of float2 (c, t) pairs,
// T = c (1 + i t) with t = tan of T's angle (c = 2^-40, t = +-2^40 where T = +-i):
//   [DIT4K_P1B1 + i]                 branch 1, pass 1: the 10 pairs of base A = W_32
//   [DIT4K_P2 + (var 16 + j) 10 + i]  pass 2, item j < 16
//   [DIT4K_P3 + (var 256 + j) 10 + i] pass 3, item j < 256
//   [DIT4K_UNP + k]                  W_8192^{-k}, k < 4096 (the unpack)
//   [DIT4K_MF + ((u 3 + t) 2 + h) 128 + 2 l], 16 bytes: the matrix-core first pass (bf16
//                                    storage, mf): lane l's A fragment of part t (three
//                                    bf16 parts) of branch u's 32 x 32 real pass-1 matrix,
//                                    K half h (layout at dit4k_table in sc_host.cpp)
// where var 0 is branch 0 (A = W_256^j, W_4096^j), var 1 branch 1 (A = W_512^{2j+1},
// W_8192^{2j+1}), var 2 the inverse (conjugates of var 0), and an item's pairs i < 10 are
// B, B^2, F_0, F_0^2, .., F_3, F_3^2 with B = A^4, F_p = A W16^p (W16^-p for the inverse).
constexpr int DIT4K_P1B1 = 0;
constexpr int DIT4K_P2 = 16;
constexpr int DIT4K_P3 = DIT4K_P2 + 3 * 16 * 10;
constexpr int DIT4K_UNP = DIT4K_P3 + 3 * 256 * 10;
constexpr int DIT4K_MF = DIT4K_UNP + 4096;
constexpr int DIT4K_TABLE_FLOAT2 = DIT4K_MF + 2 * 3 * 2 * 64 * 2;
// mf (bf16 storage only): the first pass of both branch transforms as bf16 matrix products
hipError_t launch_fused4k(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                          int head, bool pair_store, bool rev, bool mf, const float2* table,
                          hipStream_t stream);

// The fused kernels of sc_fused_dit.hip for M = 1024 and 2048 (M/2 < L <= M): passes of
// radix R1 = M/256, 16, 16 in decimation in time with tangent-merged twiddles.  Their table
// of (c, t) pairs for one M (as for the M = 4096 kernel):
//   [DIT_P1B1 + i]                     branch 1, pass 1: R1 = 4: W_8, W_8^2; R1 = 8: W_8,
//                                      W_4 (the squares) and W_16^{1+2p}, p < 4
//   [dit_p2(M) + (var R1 + k1) 10 + i]  pass 2, item k1 < R1: base W_{16 R1}^k1 (var 0),
//                                      W_{32 R1}^{2k1+1} (var 1), the conjugate of var 0 (2)
//   [dit_p3(M) + (var M/16 + m) 10 + i] pass 3, item m < M/16: W_M^m, W_2M^{2m+1}, conj
//   [dit_unp(M) + k]                   W_2M^{-k}, k < M (the unpack)
constexpr int DIT_P1B1 = 0;
constexpr int dit_p2(int) { return 6; }
constexpr int dit_p3(int M) { return dit_p2(M) + 3 * (M / 256) * 10; }
constexpr int dit_unp(int M) { return dit_p3(M) + 3 * (M / 16) * 10; }
constexpr int dit_table_size(int M) { return dit_unp(M) + M; }
hipError_t launch_fused_dit(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                            int M, int head, bool pair_store, bool rev, const float2* table,
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

// Tables of the int8 matrix-core NTT kernel (sc_ntt_mfma.hip), modulo prime A, indexed by
// lg = log2(M2) for M = 64 M2 (M2 = 1 .. 64), direction d (0 forward omega, 1 inverse omega^-1):
//   digits[d][lg]   the M2-point DFT matrix F[k][n] = omega_M2^{+-k n} zero-padded to 64 x 64,
//                   the inverse one times N^{-1} (N = 2 M), as signed base-256 digits
//                   f^(b)_a of F^(b) = 256^b F mod p, laid out [w < 4][4 a + b][lane < 64][j < 16]
//                   = f^(b)_a[16 w + lane % 16][16 (lane / 16) + j] (64 KB; digits[0][6] is
//                   also the 64-point forward matrix of the first stage)
//   inv64           the 64-point inverse matrix omega_64^{-k n} (no N^{-1}), same layout
//   twiddle[d][lg]  omega_M^{+-n2 k1} at [k1 * M2 + n2], k1 < 64, n2 < M2 (residue words)
//   roots[lg]       omega_N^i, i < N = 2 M (residue words)
struct NttMfmaTables {
    const int8_t* digits[2][7];
    const int8_t* inv64;
    const uint32_t* twiddle[2][7];
    const uint32_t* roots[7];
};

// The exact int32 convolution mod prime A with the transform stages as int8 matrix products
// (64 <= M <= 4096, one channel per workgroup); the same result bits as launch_ntt.
hipError_t launch_ntt_mfma(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch, int L,
                           int M, bool rev, const NttMfmaTables& tables, hipStream_t stream);

// Exact NTT causal convolution for FUSED_MAX_L < L <= NTT4_MAX_L through the four-step split
// (sc_ntt4.hip): M = next power of two >= L, chunks of `chunk` channels, each needing
// ntt4_bytes_per_channel(M) bytes of ws (ws_bytes >= chunk * that); wtab = the per-M tables
// of prime A (5M doubles: w_N^j for j < 2M, then the column and the row twiddles).  Modulo
// prime A, output lifted to the balanced range; rev as for launch_ntt.  Streams as for
// launch_fourstep: side null, the parts of `chunk` channels run one after the other on
// `stream` at the start of ws; with side (and fork, join), parts of chunk/2 channels
// alternate between the two streams, each with its own half of ws.
constexpr int NTT4_MAX_L = 65536;
size_t ntt4_bytes_per_channel(int M);
hipError_t launch_ntt4(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch, int L, int M,
                       bool rev, const NttTables& tables, const double* wtab, void* ws,
                       size_t ws_bytes, int64_t chunk, hipStream_t stream, hipStream_t side,
                       hipEvent_t fork, hipEvent_t join);
// The exact real-valued convolution (as launch_fixed) for FUSED_MAX_L < L <= NTT4_MAX_L
// through the same split, once per prime: tables[3] and wtab[3] (the per-M tables of primes
// A, B, C), fixed4_bytes_per_channel(M) bytes of ws per channel of a chunk; streams as for
// launch_ntt4.
size_t fixed4_bytes_per_channel(int M);
hipError_t launch_fixed4(const float* v, const float* g, float* r, int64_t nch, int L, int M,
                         int fv, int fg, const NttTables* tables, const double* const* wtab,
                         void* ws, size_t ws_bytes, int64_t chunk, hipStream_t stream,
                         hipStream_t side, hipEvent_t fork, hipEvent_t join);

// Exact real-valued causal convolution: V = round(v 2^fv), G = round(g 2^fg), the exact
// integer sum R from its residues modulo primes A, B, C (tables[0..2]), all in one kernel,
// then r = round_f32(R 2^-(fv+fg)).  Uses no scratch.
hipError_t launch_fixed(const float* v, const float* g, float* r, int64_t nch,
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
// ws holds ws_bytes >= chunk * fourstep_bytes_per_channel(M) bytes of scratch.  Without a
// second stream (side null) the channels go in parts of chunk, one after the other on
// `stream`, each reusing the start of ws.  With a second stream `side` (and two events,
// fork and join), the parts are chunk/2 channels that alternate between the two streams,
// each stream with its own half of ws: side waits for stream at the start (fork) and stream
// for side at the end (join), so the call stays ordered on `stream` as a whole.  A part
// whose scratch would end past ws_bytes is refused (hipErrorInvalidValue) before launch.
hipError_t launch_fourstep(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                           int M, int head, bool pair_store, bool rev, const float2* bank,
                           const FsTw& tw, void* ws, size_t ws_bytes, int64_t chunk,
                           hipStream_t stream, hipStream_t side, hipEvent_t fork,
                           hipEvent_t join);

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

// The allocation-free entry point's scratch: a file-scope device array of STATIC_SCRATCH_BYTES
// per device.  *ptr receives its address on the current device (looked up once per device);
// every call on a device shares it.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)64 << 20;
hipError_t static_scratch(void** ptr, size_t* bytes);

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
