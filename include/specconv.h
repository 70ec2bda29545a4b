/*
 * libspecconv -- batched per-channel causal long convolution on AMD Instinct MI355X (gfx950).
 *
 * The operation (one "channel" = one (b, c) pair, sequences of length L):
 *
 *     r[b][c][t] = sum_{j=0..t} v[b][c][j] * g[b][c][t-j],      t = 0 .. L-1
 *
 * "Caracal: Causal Architecture via Spectral Mixing" (key design 1, the multi-head Fourier
 * module) computes it as: zero-pad v and the data-dependent gate stream g on the right to
 * 2L, FFT both, multiply the spectra bin by bin, inverse FFT, keep the first L values; key
 * design 2 (the frequency-domain causal mask) explains why the truncated 2L circular
 * convolution equals this causal sum.  Every channel has its own g (the gate stream is
 * produced from the input), so nothing is shared between channels.
 *
 * "Catastrophic Token Leakage in Convolutional Sequence Modeling and How to Mitigate It"
 * (abstract) shows that float FFT convolutions leak future tokens through round-off and
 * proposes number-theoretic transforms on integers, which cannot: sc_causal_conv_ntt_i32
 * is that exact path, modulo the prime p = 998244353 (primitive root 3).
 *
 * Conventions shared by every entry point below
 * --------------------------------------------
 *  - Layout: v, g, r are dense row-major [B][C][L] arrays, t contiguous (stride 1), channel
 *    (b, c) at offset (b*C + c)*L.  B, C, L are element counts, not bytes.
 *  - Memory: v, g, r (and ws) are DEVICE pointers on the current HIP device, owned by the
 *    caller.  The library keeps no pointer after a call returns.
 *  - Asynchrony: work is enqueued on `stream` (0 = the null stream) and the call returns
 *    without waiting.  The caller keeps every buffer alive, and does not touch r, until the
 *    stream has passed the work.  Faults during execution surface at the caller's sync.
 *  - Determinism: for the same inputs and arguments the output is bitwise identical from
 *    run to run (fixed reduction order, no atomics).
 *  - Errors: status codes only; nothing is printed, no call aborts, no C++ exception crosses
 *    the boundary.  Arguments are checked on the host before any HIP call:
 *      B, C or L negative, a null pointer with B*C*L > 0, a pointer not aligned to its
 *      element size, r overlapping v or g, byte sizes overflowing int64
 *                                              -> SC_ERR_INVALID_ARGUMENT
 *      B*C*L == 0                              -> SC_OK, nothing enqueued (one exception:
 *                                                 the shared-filter gradients of an empty
 *                                                 batch, B == 0 < C*L, set dk to zero with
 *                                                 a fill kernel and need a valid dk)
 *      L above the path's maximum               -> SC_ERR_UNSUPPORTED
 *      a workspace smaller than required        -> SC_ERR_WORKSPACE
 *      a failed HIP call or kernel launch       -> SC_ERR_HIP
 *  - Library-owned state: per-device constant tables, each built by the first call on a
 *    device that needs it (a blocking host-to-device copy) and kept until the process ends:
 *    the float twiddle bank (every call), the modular tables (the first call of an exact
 *    kind: SC_KIND_NTT_I32 or SC_KIND_FIXED_F32), and the four-step tables (the first
 *    four-step call of a kind at each transform length M = next power of two >= L).  A call whose
 *    `stream` is being captured into a graph and that would have to build a table returns
 *    SC_ERR_UNSUPPORTED and enqueues nothing; sc_prepare builds them beforehand.  Also,
 *    for the four-step paths (L > 4096, every kind), a second stream and two events per
 *    device, made on first use: such a call may run half of its channel chunks on that
 *    stream, which waits for `stream` at the start of the call, and `stream` waits for it
 *    at the end, so the call stays ordered on `stream` as a whole.  While `stream` is being
 *    captured into a graph the call uses `stream` alone.  Calls from several host threads
 *    are safe.
 *  - Any L >= 1 is accepted; internally N = 2M with M the next power of two >= L.
 *    Throughput is best for powers of two.
 *  - Inputs of the float paths must be finite.  (A NaN or Inf at v_s reaches every output of
 *    its channel through the transform, including t < s, whereas the causal sum would only
 *    reach t >= s.)
 */
#ifndef SPECCONV_H
#define SPECCONV_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sc_status {
    SC_OK = 0,
    SC_ERR_INVALID_ARGUMENT = 1,
    SC_ERR_UNSUPPORTED = 2,
    SC_ERR_HIP = 3,
    SC_ERR_WORKSPACE = 4
} sc_status;

typedef enum sc_kind {
    SC_KIND_F32 = 0,      /* float32 storage, float32 arithmetic                    */
    SC_KIND_BF16 = 1,     /* bfloat16 storage, float32 arithmetic                   */
    SC_KIND_NTT_I32 = 2,  /* int32 storage, exact arithmetic in Z_p, p = 998244353   */
    SC_KIND_FIXED_F32 = 3 /* float32 storage, exact arithmetic on fixed-point
                             encodings (see sc_causal_conv_fixed_f32)               */
} sc_kind;

typedef enum sc_path {
    SC_PATH_AUTO = 0,      /* the library's choice (below)                         */
    SC_PATH_FUSED = 1,     /* one workgroup per channel, transform held in LDS     */
    SC_PATH_FOUR_STEP = 2, /* column / twiddle / row transforms staged through HBM  */
    SC_PATH_DIRECT = 3,    /* direct fp32 summation (float kinds, small L only)     */
    SC_PATH_NTT_MFMA = 4,  /* SC_KIND_NTT_I32, L <= 4096: the transform stages as int8
                              matrix products on the matrix cores (the integer-matrix
                              formulation of "Catastrophic Token Leakage ...", abstract);
                              the same result bits as SC_PATH_FUSED                  */
    SC_PATH_FUSED_MFMA = 5 /* SC_KIND_BF16, 2048 < L <= 4096: SC_PATH_FUSED with the first
                              radix-16 pass of each branch transform (the pad-2L FFT of
                              the Caracal notes, key designs 1-2) as bf16 matrix products
                              on the matrix cores, exact products of the bf16 inputs and
                              a three-part bf16 DFT matrix summed in fp32; the same
                              accuracy bound, not the same bits.  No faster than
                              SC_PATH_FUSED on MI355X (within a few percent either
                              way; kept for measurement)                              */
} sc_path;

/* Optional controls for sc_causal_conv_ex (testing and experiments). */
typedef struct sc_options {
    int32_t path;      /* sc_path; SC_PATH_AUTO picks: L <= 32 direct, L <= 4096 fused,
                          larger L four-step (the exact kinds: fused up to 4096,
                          four-step up to 65536)                                     */
    int32_t head;      /* float kinds: outputs t < head are computed by direct fp32
                          summation instead of the transform.  -1 = default (32);
                          0 disables; odd values are rounded up to even; at most 64.  */
    int32_t frac_v;    /* SC_KIND_FIXED_F32: fraction bits fv of v's encoding, in
                          [-64, 64]; must be 0 for the other kinds                   */
    int32_t frac_g;    /* likewise fg for g                                          */
    int32_t reserved[4]; /* must be zero */
} sc_options;

/*
 * sc_causal_conv_f32 -- r = causal_conv(v, g), float32 in and out.
 *   Pad-to-2L FFT method of the Caracal notes (key designs 1-2) in fp32 arithmetic.
 *   Accuracy: |r_t - exact_t| <= 1e-4 * sum_{j<=t} |v_j||g_{t-j}| for the inputs this
 *   library is tested on (the first 32 outputs use direct summation).
 *   L <= 4096 runs fused in LDS and allocates nothing.  L > 4096 uses the four-step path,
 *   which needs sc_workspace_bytes(SC_KIND_F32, B, C, L) bytes of device scratch; this call
 *   allocates it stream-ordered on `stream` (hipMallocAsync/hipFreeAsync).  Use
 *   sc_causal_conv_f32_ws to supply it instead.  Largest L: 4,194,304.
 */
sc_status sc_causal_conv_f32(const float* v, const float* g, float* r, int64_t B, int64_t C,
                             int64_t L, hipStream_t stream);

/*
 * sc_causal_conv_bf16 -- as sc_causal_conv_f32 with bfloat16 storage.
 *   v, g, r hold bfloat16 bit patterns (uint16_t).  Inputs are widened exactly to fp32,
 *   all arithmetic is fp32, and each output is rounded once to bfloat16 (nearest, ties to
 *   even).  Accuracy: the fp32 bound plus one bf16 rounding, 2^-8 |r_t|.
 */
sc_status sc_causal_conv_bf16(const uint16_t* v, const uint16_t* g, uint16_t* r, int64_t B,
                              int64_t C, int64_t L, hipStream_t stream);

/*
 * sc_causal_conv_ntt_i32 -- exact causal convolution of int32 sequences through a
 *   number-theoretic transform modulo p = 998244353 ("Catastrophic Token Leakage ...",
 *   abstract: an FFT executed on integers only, which provably leaks no future token).
 *   Inputs are reduced into Z_p (x < 0 -> x + p after reduction).  Output:
 *       r_t = the residue of sum_{j<=t} v_j g_{t-j} mod p, in [-(p-1)/2, (p-1)/2].
 *   It equals the integer sum whenever |sum| <= (p-1)/2 = 499,122,176: a caller
 *   precondition (see sc_ntt_range_ok).  Output t depends on v_0..v_t, g_0..g_t only, bit
 *   for bit.  L <= 4096: the transform is held in LDS, no allocation.  4096 < L <= 65536:
 *   the four-step split (column transforms, rows of 4096 in LDS, inverse columns) through
 *   scratch of 24 M bytes per channel in chunks (sc_workspace_bytes(SC_KIND_NTT_I32, ...)),
 *   allocated stream-ordered by this call; the _ws variant takes it from the caller.
 *   Largest L: 65536.
 */
sc_status sc_causal_conv_ntt_i32(const int32_t* v, const int32_t* g, int32_t* r, int64_t B,
                                 int64_t C, int64_t L, hipStream_t stream);

/*
 * sc_causal_conv_fixed_f32 -- exactly causal convolution of float32 data ("Catastrophic
 *   Token Leakage ...", abstract: a number-theoretic FFT on integers leaks no future token;
 *   here real activations reach the integers through a fixed-point encoding whose scales
 *   the caller fixes, so no scale depends on the data):
 *       V_j = round(v_j 2^frac_v),  G_j = round(g_j 2^frac_g)     (nearest, ties to even)
 *       R_t = sum_{j<=t} V_j G_{t-j}                              (exact integer)
 *       r_t = R_t 2^-(frac_v + frac_g) rounded once to float32    (nearest, ties to even,
 *                                                                  subnormals included)
 *   R_t is computed exactly with the pad-2L recipe modulo three primes (998244353,
 *   1004535809, 469762049) and the Chinese remainder theorem, so output t depends on
 *   v_0..v_t and g_0..g_t alone, bit for bit, and equals the definition above whenever
 *   |V_j|, |G_j| < 2^51 and |R_t| <= (p_A p_B p_C - 1) / 2 (about 2^87.6): a caller
 *   precondition, checked from bounds by sc_fixed_range_ok.  Accuracy against the real sum:
 *   |r_t - sum v_j g_{t-j}| <= 2^-(frac_v+1) sum_j |g_j| + 2^-(frac_g+1) sum_j |v_j| + (one
 *   float32 rounding) -- e.g. frac_v = frac_g = 24 for activations of magnitude below 8.
 *   frac_v, frac_g in [-64, 64].  Largest L: 65536.  L <= 4096: one kernel computes the
 *   three residues of each output in turn and combines them: no scratch, no allocation
 *   (sc_workspace_bytes is 0 there; the _ws variant then accepts any ws and ws_bytes and
 *   uses neither).  4096 < L <= 65536: the four-step split of sc_causal_conv_ntt_i32, run
 *   once per prime, then one kernel that recombines the three residues of each output;
 *   it needs sc_workspace_bytes(SC_KIND_FIXED_F32, B, C, L) bytes of device scratch (40 M
 *   bytes per channel of a chunk, M = the power of two >= L), allocated stream-ordered on
 *   `stream` by this call, or supplied through the _ws variant.  Gradients are not offered
 *   for this kind (SC_ERR_UNSUPPORTED from sc_causal_conv_bwd_ex).
 */
sc_status sc_causal_conv_fixed_f32(const float* v, const float* g, float* r, int64_t B,
                                   int64_t C, int64_t L, int32_t frac_v, int32_t frac_g,
                                   hipStream_t stream);
sc_status sc_causal_conv_fixed_f32_ws(const float* v, const float* g, float* r, int64_t B,
                                      int64_t C, int64_t L, int32_t frac_v, int32_t frac_g,
                                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sc_fixed_range_ok -- 1 if |v_j| <= max_abs_v and |g_j| <= max_abs_g guarantee the
 *   preconditions of sc_causal_conv_fixed_f32 for these fraction bits and L (encodings below
 *   2^51, L * max|V| * max|G| <= (p_A p_B p_C - 1) / 2); 0 otherwise.  Host only.
 */
int sc_fixed_range_ok(double max_abs_v, double max_abs_g, int32_t frac_v, int32_t frac_g,
                      int64_t L);

/*
 * sc_workspace_bytes -- device scratch bytes a call of this kind and shape needs
 *   (0 when the chosen path needs none, e.g. the fused path).  Returns 0 for invalid
 *   arguments as well.
 */
size_t sc_workspace_bytes(sc_kind kind, int64_t B, int64_t C, int64_t L);

/*
 * sc_causal_conv_*_ws -- as above, with caller-owned scratch: ws (device pointer, 256-byte
 *   aligned) of ws_bytes bytes.  ws_bytes below sc_workspace_bytes(...) -> SC_ERR_WORKSPACE.
 *   ws may be null when the requirement is 0.  The library never allocates in these calls.
 *   The caller keeps ws alive and unshared until the stream has passed the work.
 */
sc_status sc_causal_conv_f32_ws(const float* v, const float* g, float* r, int64_t B, int64_t C,
                                int64_t L, void* ws, size_t ws_bytes, hipStream_t stream);
sc_status sc_causal_conv_bf16_ws(const uint16_t* v, const uint16_t* g, uint16_t* r, int64_t B,
                                 int64_t C, int64_t L, void* ws, size_t ws_bytes,
                                 hipStream_t stream);
sc_status sc_causal_conv_ntt_i32_ws(const int32_t* v, const int32_t* g, int32_t* r, int64_t B,
                                    int64_t C, int64_t L, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/*
 * sc_causal_conv_ex -- any kind, with options (opt may be null = defaults) and an optional
 *   caller workspace (ws null and ws_bytes 0: allocate stream-ordered when needed).
 *   v, g, r point to elements of the kind's storage type.  A path that cannot serve the
 *   kind and L -> SC_ERR_UNSUPPORTED; nonzero reserved fields, or nonzero frac_v/frac_g for
 *   a kind other than SC_KIND_FIXED_F32 -> SC_ERR_INVALID_ARGUMENT.
 */
sc_status sc_causal_conv_ex(sc_kind kind, const void* v, const void* g, void* r, int64_t B,
                            int64_t C, int64_t L, const sc_options* opt, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * Token-major layout.  In the Caracal layer v and g are linear projections (for g, followed
 * by a grouped convolution) of the normalised activations ("Caracal: Causal Architecture
 * via Spectral Mixing", key design 1), so a model holds them token-major, (B, L, C):
 * element (b, t, c) at (b L + t) C + c.  These calls take v, g and r in that layout and
 * compute the same r as sc_causal_conv_* (every kind and path, same accuracy and limits;
 * the argument order B, L, C follows the layout).  They move a chunk of channels at a
 * time into channel rows in a staging workspace, run the ordinary kernels there and move
 * the result back, so no caller transpose of the whole tensors is needed.
 *
 *  sc_blc_workspace_bytes(kind, B, L, C) -- bytes of that workspace (three staging buffers
 *      of at most 32 MiB each, plus the path's own scratch for one chunk); 0 for invalid
 *      arguments or an empty call.
 *  sc_causal_conv_blc_f32 / _bf16 -- allocate the workspace stream-ordered
 *      (hipMallocAsync / hipFreeAsync on `stream`).
 *  sc_causal_conv_blc_ex -- any kind, with options as sc_causal_conv_ex and a caller
 *      workspace: ws null (the call allocates) with ws_bytes 0, or a 256-byte aligned
 *      device buffer of at least sc_blc_workspace_bytes(kind, B, L, C) bytes (else
 *      SC_ERR_WORKSPACE) that overlaps none of v, g, r (else SC_ERR_INVALID_ARGUMENT).
 *
 * r may not overlap v or g.  Errors as sc_causal_conv_ex.
 */
size_t sc_blc_workspace_bytes(sc_kind kind, int64_t B, int64_t L, int64_t C);
sc_status sc_causal_conv_blc_f32(const float* v, const float* g, float* r, int64_t B, int64_t L,
                                 int64_t C, hipStream_t stream);
sc_status sc_causal_conv_blc_bf16(const uint16_t* v, const uint16_t* g, uint16_t* r, int64_t B,
                                  int64_t L, int64_t C, hipStream_t stream);
sc_status sc_causal_conv_blc_ex(sc_kind kind, const void* v, const void* g, void* r, int64_t B,
                                int64_t L, int64_t C, const sc_options* opt, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/*
 * Gate stream.  The Caracal layer makes each channel's convolution kernel from the input
 * ("Caracal: Causal Architecture via Spectral Mixing", key design 1): g = Conv1d_G2(sigma(s)),
 * s a linear projection of the normalised activations, Conv1d_G2 a causal convolution with
 * kernel 3 grouped by head (64 channels per group), so that
 *
 *     g[b][co][t] = sum_{i<64} sum_{k<3} W[co][i][k] * sigmoid(s[b][c0+i][t+k-2])
 *
 * with c0 = 64 * (co / 64), the convolution's input zero before t = 0 (left padding 2),
 * W of shape (C, 64, 3) row-major (PyTorch's Conv1d weight with groups = C / 64).  The
 * contraction runs on the matrix cores with fp32 accumulation; bfloat16 storage rounds
 * sigmoid(s) to bfloat16 before the product (the precision a bfloat16 layer computes it in)
 * and g once at the end.  C must be a multiple of 64 (else SC_ERR_UNSUPPORTED); W must be
 * 16-byte aligned (else SC_ERR_INVALID_ARGUMENT).
 *
 *  sc_gate_f32 / _bf16(s, W, g, B, C, L, stream) -- g from s, both channel-major (B, C, L).
 *      g may overlap neither s nor W.  Allocates nothing.
 *  sc_gate_conv_ex(kind, v, s, W, r, B, C, L, opt, ws, ws_bytes, stream) -- the layer's
 *      mixing step r = causal_conv(v, gate(s, W)) with v, s, r channel-major: g is made
 *      chunk by chunk into the workspace (sc_gate_conv_workspace_bytes; ws null with
 *      ws_bytes 0 allocates it stream-ordered) and never written to r's side of memory.
 *  sc_gate_conv_blc_ex / _f32 / _bf16 -- the same with v, s, r token-major (B, L, C), as in
 *      a model: per chunk v is moved into channel rows, g made from s straight into channel
 *      rows, convolved and moved back (sc_gate_conv_blc_workspace_bytes; the _f32 / _bf16
 *      calls allocate).  s must be 16-byte aligned.
 * kind is SC_KIND_F32 or SC_KIND_BF16; opt, ws and the convolution's limits and accuracy as
 * sc_causal_conv_ex / sc_causal_conv_blc_ex, for g as computed here.  r may not overlap v, s
 * or W.  Errors as sc_causal_conv_ex.
 */
sc_status sc_gate_f32(const float* s, const float* W, float* g, int64_t B, int64_t C, int64_t L,
                      hipStream_t stream);
sc_status sc_gate_bf16(const uint16_t* s, const uint16_t* W, uint16_t* g, int64_t B, int64_t C,
                       int64_t L, hipStream_t stream);
size_t sc_gate_conv_workspace_bytes(sc_kind kind, int64_t B, int64_t C, int64_t L);
size_t sc_gate_conv_blc_workspace_bytes(sc_kind kind, int64_t B, int64_t L, int64_t C);
sc_status sc_gate_conv_ex(sc_kind kind, const void* v, const void* s, const void* W, void* r,
                          int64_t B, int64_t C, int64_t L, const sc_options* opt, void* ws,
                          size_t ws_bytes, hipStream_t stream);
sc_status sc_gate_conv_blc_ex(sc_kind kind, const void* v, const void* s, const void* W, void* r,
                              int64_t B, int64_t L, int64_t C, const sc_options* opt, void* ws,
                              size_t ws_bytes, hipStream_t stream);
sc_status sc_gate_conv_blc_f32(const float* v, const float* s, const float* W, float* r,
                               int64_t B, int64_t L, int64_t C, hipStream_t stream);
sc_status sc_gate_conv_blc_bf16(const uint16_t* v, const uint16_t* s, const uint16_t* W,
                                uint16_t* r, int64_t B, int64_t L, int64_t C, hipStream_t stream);

/*
 * Gradients (backward pass).  The Caracal models are trained end to end with a next-token
 * loss ("Caracal: Causal Architecture via Spectral Mixing", loss function / training
 * strategy), so the convolution of key design 1 needs its vector-Jacobian product: for the
 * output gradient dr = dLoss/dr (same layout as r),
 *
 *     dv[b][c][j] = sum_{t=j..L-1} dr[b][c][t] * g[b][c][t-j]
 *     dg[b][c][k] = sum_{t=k..L-1} dr[b][c][t] * v[b][c][t-k]
 *
 * i.e. dv = rev(causal_conv(rev(dr), g)) and dg = rev(causal_conv(rev(dr), v)), where rev
 * reverses t.  The library computes each as a causal convolution on the same paths as the
 * forward call (the first input read reversed, the output written reversed): same pad-2L
 * transform, same accuracy statement with the error scale
 *     sum_{t>=j} |dr_t| |g_{t-j}|   (for dv)   and   sum_{t>=k} |dr_t| |v_{t-k}|   (for dg),
 * and the last 32 outputs (j >= L-32), whose scale holds few products, by direct fp32
 * summation.  The exact kind returns the residues of the two sums mod p in the symmetric
 * range; dv_j depends on dr_j..dr_{L-1} only, bit for bit.
 *
 * Arguments: dr, v, g as in the forward call; dv, dg are outputs of the same shape, and may
 * overlap neither each other nor any input (-> SC_ERR_INVALID_ARGUMENT).  The other
 * conventions, limits and errors are those of the forward call of the same kind.  Scratch:
 * the two gradients run one after the other and share one workspace, so a call needs
 * sc_workspace_bytes(kind, B, C, L) bytes, the same as the forward call of that shape.
 */
sc_status sc_causal_conv_bwd_f32(const float* dr, const float* v, const float* g, float* dv,
                                 float* dg, int64_t B, int64_t C, int64_t L, hipStream_t stream);
sc_status sc_causal_conv_bwd_bf16(const uint16_t* dr, const uint16_t* v, const uint16_t* g,
                                  uint16_t* dv, uint16_t* dg, int64_t B, int64_t C, int64_t L,
                                  hipStream_t stream);
sc_status sc_causal_conv_bwd_ntt_i32(const int32_t* dr, const int32_t* v, const int32_t* g,
                                     int32_t* dv, int32_t* dg, int64_t B, int64_t C, int64_t L,
                                     hipStream_t stream);
/* any kind, with options and an optional caller workspace, as sc_causal_conv_ex */
sc_status sc_causal_conv_bwd_ex(sc_kind kind, const void* dr, const void* v, const void* g,
                                void* dv, void* dg, int64_t B, int64_t C, int64_t L,
                                const sc_options* opt, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * Filter shared by the batch.  The Caracal notes contrast their data-dependent gate with
 * filters that do not depend on the input ("Caracal: Causal Architecture via Spectral
 * Mixing", related work: Hyena's position-based filter, FlashButterfly's static global
 * kernel).  For such a filter k[C][L] (one per channel, the same for every batch row):
 *
 *     r[b][c][t] = sum_{j=0..t} v[b][c][j] * k[c][t-j]
 *
 * by the same pad-2L method, with the filter's spectrum computed once (and reusable across
 * calls) and two batch rows sharing one complex transform (k is real, so the transform of
 * v_b + i v_{b+1} times K gives both rows).  Accuracy as sc_causal_conv_f32 / _bf16 with
 * g_{t-j} = k_{t-j}; the first 32 outputs use direct fp32 summation.  1 <= L <= 4096 (else
 * SC_ERR_UNSUPPORTED), C * L elements of k, and the whole batch of v and r, processed in
 * launches of at most 2^31 bytes of rows each; C * L * element size must stay below 2^31
 * bytes (SC_ERR_UNSUPPORTED otherwise).  Float kinds only.
 *
 *  sc_filter_spectrum_bytes(C, L) -- bytes of the spectrum of C filters of length L
 *      (C * (2M + 32) * 8 with M = max(64, next power of two >= L)); 0 for unsupported L.
 *  sc_filter_spectrum_*(k, spec, C, L, stream) -- writes that spectrum (device memory
 *      owned by the caller, 8-byte aligned, not overlapping k).  Its contents are private
 *      to this library version; it is valid for this C and L only.
 *  sc_causal_conv_spec_*(v, spec, r, B, C, L, stream) -- r from v and a spectrum made for
 *      the same C and L.  r may not overlap v or spec.  Allocates nothing.
 *  sc_causal_conv_shared_*(v, k, r, B, C, L, stream) -- both steps in one call, the
 *      spectrum in stream-ordered scratch (hipMallocAsync / hipFreeAsync on `stream`).
 */
size_t sc_filter_spectrum_bytes(int64_t C, int64_t L);
sc_status sc_filter_spectrum_f32(const float* k, void* spec, int64_t C, int64_t L,
                                 hipStream_t stream);
sc_status sc_filter_spectrum_bf16(const uint16_t* k, void* spec, int64_t C, int64_t L,
                                  hipStream_t stream);
sc_status sc_causal_conv_spec_f32(const float* v, const void* spec, float* r, int64_t B,
                                  int64_t C, int64_t L, hipStream_t stream);
sc_status sc_causal_conv_spec_bf16(const uint16_t* v, const void* spec, uint16_t* r, int64_t B,
                                   int64_t C, int64_t L, hipStream_t stream);
sc_status sc_causal_conv_shared_f32(const float* v, const float* k, float* r, int64_t B,
                                    int64_t C, int64_t L, hipStream_t stream);
sc_status sc_causal_conv_shared_bf16(const uint16_t* v, const uint16_t* k, uint16_t* r,
                                     int64_t B, int64_t C, int64_t L, hipStream_t stream);

/*
 * Gradients for a filter shared by the batch, for the output gradient dr (as r):
 *     dv[b][c][j] = sum_{t=j..L-1} dr[b][c][t] k[c][t-j]
 *     dk[c][j]    = sum_b sum_{t=j..L-1} dr[b][c][t] v[b][c][t-j]
 * dv by the apply kernel run on dr reversed (with the filter's spectrum: the _spec_ calls
 * take one made by sc_filter_spectrum_* for this C and L, the _shared_ calls make it in
 * stream-ordered scratch), dk by a kernel that sums the spectral products over the batch
 * rows and inverts once per channel.  Accuracy as the forward calls with the error scales
 * sum_t |dr_t||k_{t-j}| and sum_b sum_t |dr_t||v_{t-j}|; the last 32 positions of dv and dk
 * use direct fp32 summation.  dv (B*C*L elements) and dk (C*L) may overlap neither each
 * other nor dr, v, k or the spectrum.  With B = 0 (and C*L > 0) only dk is touched: it is
 * set to zero, the sum over no rows.  Limits and errors as sc_causal_conv_shared_*.
 */
sc_status sc_causal_conv_spec_bwd_f32(const float* dr, const float* v, const void* spec,
                                      float* dv, float* dk, int64_t B, int64_t C, int64_t L,
                                      hipStream_t stream);
sc_status sc_causal_conv_spec_bwd_bf16(const uint16_t* dr, const uint16_t* v, const void* spec,
                                       uint16_t* dv, uint16_t* dk, int64_t B, int64_t C,
                                       int64_t L, hipStream_t stream);
sc_status sc_causal_conv_shared_bwd_f32(const float* dr, const float* v, const float* k, float* dv,
                                        float* dk, int64_t B, int64_t C, int64_t L,
                                        hipStream_t stream);
sc_status sc_causal_conv_shared_bwd_bf16(const uint16_t* dr, const uint16_t* v, const uint16_t* k,
                                         uint16_t* dv, uint16_t* dk, int64_t B, int64_t C,
                                         int64_t L, hipStream_t stream);

/*
 * sc_ntt_range_ok -- 1 if every |v_j| <= max_abs_v and |g_j| <= max_abs_g guarantee that
 *   the exact sums fit the symmetric residue range, i.e. L * max_abs_v * max_abs_g <=
 *   (p-1)/2; 0 otherwise (or on negative arguments).  Host only.
 */
int sc_ntt_range_ok(int64_t max_abs_v, int64_t max_abs_g, int64_t L);

/* Human-readable name of a status code (static storage).  Host only. */
const char* sc_status_string(sc_status s);

/*
 * sc_causal_conv_noalloc -- sc_causal_conv_ex(kind, v, g, r, B, C, L, NULL, ...) for the
 *   kinds SC_KIND_F32, SC_KIND_BF16 and SC_KIND_NTT_I32, for callers that cannot allocate
 *   device memory (code under graph capture, tight serving loops, harnesses that forbid
 *   allocation).  The call allocates nothing and creates nothing: the scratch of the
 *   four-step path (L > 4096) is a static device array of SC_NOALLOC_SCRATCH_BYTES, one per
 *   GPU, held from the library's load until the process ends; the call stays on `stream`
 *   (no second stream); the constant tables must already exist on the device (made by
 *   sc_prepare(kind, L) or by any earlier call of that kind and transform length),
 *   otherwise SC_ERR_UNSUPPORTED and nothing is enqueued.  A length whose four-step scratch
 *   for one channel exceeds SC_NOALLOC_SCRATCH_BYTES (L > 2,097,152) is SC_ERR_UNSUPPORTED;
 *   more channels than the array holds at once run as several parts on `stream`.
 *   SC_KIND_FIXED_F32 is SC_ERR_INVALID_ARGUMENT.  Results are bitwise those of
 *   sc_causal_conv_ex with the same arguments.  Every call on one GPU uses the same array:
 *   calls that may overlap on one GPU (other streams, other host threads) race and must be
 *   ordered by the caller.
 */
#define SC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sc_status sc_causal_conv_noalloc(sc_kind kind, const void* v, const void* g, void* r, int64_t B,
                                 int64_t C, int64_t L, hipStream_t stream);

/*
 * sc_prepare -- builds, on the current device, every constant table that a call of this
 *   kind and length needs (see "Library-owned state" above), so that such calls can then be
 *   captured into a graph.  Blocking (host-to-device copies on the null stream); call it
 *   outside any capture.  Returns SC_ERR_UNSUPPORTED for a length the kind does not support,
 *   SC_ERR_INVALID_ARGUMENT for a bad kind or L < 0, SC_ERR_HIP if an allocation or copy
 *   fails; L == 0 needs no table (SC_OK, nothing done).  Safe to call repeatedly and from
 *   several host threads.
 */
sc_status sc_prepare(sc_kind kind, int64_t L);

/* Library version: major * 10000 + minor * 100 + patch (this header: 902).  Host only. */
int sc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECCONV_H */
