// libspecconv host layer: argument checks, per-device constant tables, path choice and
// kernel launches behind the C ABI declared in include/specconv.h.
#include "specconv.h"

#include <climits>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "sc_internal.h"

static_assert(SC_NOALLOC_SCRATCH_BYTES == sc::STATIC_SCRATCH_BYTES,
              "the header states the static scratch size");

namespace {

constexpr int kMaxDevices = 64;
constexpr int kDefaultHead = 32;
constexpr int kMaxHead = 64;
constexpr int64_t kMaxLFused = 4096;     // fused path; longer sequences use the four-step path
constexpr int64_t kMinLFourStep = 2049;  // the four-step split needs M >= 4096
// channels per four-step chunk: as many as fit this much scratch (enough channels to
// fill the GPU in every kernel of a half chunk; measured best among 128..256 MB with the
// halves on two streams, and among 24..384 MB on one)
#ifndef SC_FS_CHUNK_MB
#define SC_FS_CHUNK_MB 192
#endif
constexpr int64_t kFourStepChunkBytes = (int64_t)SC_FS_CHUNK_MB << 20;
constexpr int64_t kMaxLNtt = 4096;
// M = 4096 float convolutions use the kernel of sc_fused4k.hip (0: the general fused kernel)
#ifndef SC_FUSED4K
#define SC_FUSED4K 1
#endif
constexpr bool kFused4k = SC_FUSED4K != 0;
// M = 1024 and 2048 float convolutions use the kernels of sc_fused_dit.hip (0: the general
// fused kernel)
#ifndef SC_FUSED_DIT
#define SC_FUSED_DIT 1
#endif
constexpr bool kFusedDit = SC_FUSED_DIT != 0;
constexpr int64_t kNttP = 998244353;
constexpr int32_t kMaxFrac = 64;          // |fixed-point fraction bits| of the exact real kind
// the shared-filter gradients take the one-kernel path when it has at least this many
// workgroups (its row loop runs per channel group; fewer groups leave CUs idle)
constexpr int64_t kSharedBwdMinBlocks = 512;

sc_status upload(const void* host, size_t bytes, void** dev)
{
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) return SC_ERR_HIP;
    if (hipMemcpy(p, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(p);
        return SC_ERR_HIP;
    }
    *dev = p;
    return SC_OK;
}

struct DeviceState {
    float2* fused_tw = nullptr;   // the float twiddle bank (sc_internal.h)
    float2* dit4k = nullptr;      // the M = 4096 fused kernel's (c, t) table (sc_internal.h)
    float2* dit[2] = {nullptr, nullptr};   // the M = 1024, 2048 kernels' tables (sc_internal.h)
    sc::NttTables ntt[3]{};       // primes A, B, C (sc::NTT_PRIMES)
    bool ntt_ready = false;
    sc::NttMfmaTables mfma{};     // the matrix-core NTT kernel's tables (prime A)
    bool mfma_ready = false;
    std::map<int, sc::FsTw> fs;     // four-step tables by M
    std::map<std::pair<int, int>, const double*> ntt4;   // four-step NTT tables by (M, prime)
    // the four-step path's second stream (default priority, non-blocking) and its fork/join
    // events; fs_mu keeps one call's fork, launches and join together, since the events are
    // shared by every call on the device
    hipStream_t fs_side = nullptr;
    hipEvent_t fs_fork = nullptr, fs_join = nullptr;
    std::mutex fs_mu;
};

uint64_t powmod(uint64_t b, uint64_t e, uint64_t m)
{
    uint64_t r = 1;
    b %= m;
    while (e) {
        if (e & 1) r = (uint64_t)((unsigned __int128)r * b % m);
        b = (uint64_t)((unsigned __int128)b * b % m);
        e >>= 1;
    }
    return r;
}

sc_status build_ntt_tables(sc::NttTables* t, uint64_t p)
{
    std::vector<double> h(2 * (size_t)sc::NTT_BANK_ENTRIES);
    auto put = [&](size_t i, uint64_t w) {
        h[2 * i] = (double)w;
        h[2 * i + 1] = (double)w / (double)p;
    };
    const uint64_t w8192 = powmod(3, (p - 1) / sc::NTT_TW_N, p);
    uint64_t x = 1;
    for (int i = 0; i < sc::NTT_TW_N; ++i) {
        put((size_t)i, x);
        x = x * w8192 % p;
    }
    for (int Q = 32; Q <= 4096; Q *= 2) {
        const uint64_t wq = powmod(3, (p - 1) / (uint64_t)Q, p);
        for (int k = 0; k < 16; ++k)
            for (int n = 0; n < Q / 16; ++n)
                put((size_t)(sc::NTT_PASS_BASE + (Q - 32) + k * (Q / 16) + n),
                    powmod(wq, (uint64_t)n * (uint64_t)k, p));
    }
    void* d = nullptr;
    sc_status st = upload(h.data(), h.size() * sizeof(double), &d);
    if (st != SC_OK) return st;
    t->bank = (const double*)d;
    for (int k = 0; k < 24; ++k) {
        const uint64_t ninv = powmod(powmod(2, (uint64_t)k, p), p - 2, p);
        t->ninv[k] = (double)ninv;
        t->ninv_q[k] = (double)ninv / (double)p;
    }
    return SC_OK;
}

// The int8 matrix-core NTT kernel's tables (layouts in sc_internal.h), one upload.
sc_status build_mfma_tables(sc::NttMfmaTables* t)
{
    const uint64_t p = sc::NTT_PRIMES[0];
    const size_t digit_bytes = 4 * 16 * 64 * 16;   // per matrix
    size_t ntw = 0, nroot = 0;
    for (int lg = 0; lg <= 6; ++lg) {
        ntw += 2 * (size_t)64 * ((size_t)1 << lg);
        nroot += (size_t)128 << lg;
    }
    const size_t dbytes = 15 * digit_bytes;   // 7 forward, 7 scaled inverse, the 64-point inverse
    std::vector<unsigned char> h(dbytes + (ntw + nroot) * sizeof(uint32_t));
    int8_t* dig = (int8_t*)h.data();
    uint32_t* tw = (uint32_t*)(h.data() + dbytes);
    size_t toff[2][7], roff[7], pos = 0;
    for (int d = 0; d < 2; ++d)
        for (int lg = 0; lg <= 6; ++lg) {
            toff[d][lg] = pos;
            pos += (size_t)64 << lg;
        }
    for (int lg = 0; lg <= 6; ++lg) {
        roff[lg] = pos;
        pos += (size_t)128 << lg;
    }
    for (int d = 0; d < 2; ++d)
        for (int lg = 0; lg <= 7; ++lg) {
            if (d == 0 && lg == 7) continue;
            // lg 7: the plain 64-point inverse matrix
            const uint64_t M2 = (uint64_t)1 << (lg == 7 ? 6 : lg), M = 64 * M2;
            const bool scaled = d == 1 && lg < 7;
            // the M2-point DFT matrix (zero-padded; the inverse times N^{-1} except at lg 7),
            // then the digits of 256^b F mod p
            const uint64_t wm2 = powmod(3, (p - 1) / M2, p);
            const uint64_t w2 = d ? powmod(wm2, p - 2, p) : wm2;
            const uint64_t scale = scaled ? powmod(2 * M % p, p - 2, p) : 1;
            int8_t* out = dig + (size_t)(lg == 7 ? 14 : d * 7 + lg) * digit_bytes;
            for (uint64_t k = 0; k < 64; ++k)
                for (uint64_t n = 0; n < 64; ++n) {
                    const uint64_t f =
                        (k < M2 && n < M2) ? powmod(w2, k * n, p) * scale % p : 0;
                    const int w = (int)(k / 16), lane = (int)(k % 16 + 16 * (n / 16));
                    const int j = (int)(n % 16);
                    uint64_t fb = f;   // 256^b F mod p
                    for (int b = 0; b < 4; ++b, fb = fb * 256 % p) {
                        // balanced base-256 digits: fb = sum_a dg_a 256^a, dg in [-128, 127]
                        int64_t y = (int64_t)fb;
                        for (int a = 0; a < 4; ++a) {
                            int dg = (int)(y & 255);
                            if (dg >= 128) dg -= 256;
                            y = (y - dg) >> 8;
                            out[(((size_t)w * 16 + 4 * a + b) * 64 + lane) * 16 + j] = (int8_t)dg;
                        }
                    }
                }
            if (lg == 7) continue;
            // twiddles omega_M^{+-n2 k1}
            const uint64_t wm = powmod(3, (p - 1) / M, p);
            const uint64_t wt = d ? powmod(wm, p - 2, p) : wm;
            for (uint64_t k1 = 0; k1 < 64; ++k1)
                for (uint64_t n2 = 0; n2 < M2; ++n2)
                    tw[toff[d][lg] + k1 * M2 + n2] = (uint32_t)powmod(wt, k1 * n2, p);
        }
    for (int lg = 0; lg <= 6; ++lg) {
        const uint64_t N = (uint64_t)128 << lg;
        const uint64_t wn = powmod(3, (p - 1) / N, p);
        uint64_t x = 1;
        for (uint64_t i = 0; i < N; ++i) {
            tw[roff[lg] + i] = (uint32_t)x;
            x = x * wn % p;
        }
    }
    void* dev = nullptr;
    const sc_status st = upload(h.data(), h.size(), &dev);
    if (st != SC_OK) return st;
    const unsigned char* base = (const unsigned char*)dev;
    const uint32_t* tb = (const uint32_t*)(base + dbytes);
    for (int d = 0; d < 2; ++d)
        for (int lg = 0; lg <= 6; ++lg) {
            t->digits[d][lg] = (const int8_t*)(base + (size_t)(d * 7 + lg) * digit_bytes);
            t->twiddle[d][lg] = tb + toff[d][lg];
        }
    t->inv64 = (const int8_t*)(base + 14 * digit_bytes);
    for (int lg = 0; lg <= 6; ++lg) t->roots[lg] = tb + roff[lg];
    return SC_OK;
}

// T = c (1 + i t) for the unit root exp(-2 pi i e / n) (conjugated when inv), computed in
// float64 and rounded once per component; c = 2^-40, t = +-2^40 stand in for c = 0
float2 tan_pair(double e, double n, bool inv)
{
    const double a = 6.283185307179586476925286766559 * e / n;
    const double c = std::cos(a), s = (inv ? 1.0 : -1.0) * std::sin(a);
    if (std::fabs(c) < 0x1p-30) return make_float2(0x1p-40f, (float)(s * 0x1p40));
    return make_float2((float)c, (float)(s / c));
}

// the pairs B, B^2, F_0, F_0^2, .., F_3, F_3^2 of a radix-16 item with twiddle base
// A = exp(-+2 pi i a / n): B = A^4, F_p = A W16^{+-p}
void item_pairs(float2* out, double a, double n, bool inv)
{
    out[0] = tan_pair(4 * a, n, inv);
    out[1] = tan_pair(8 * a, n, inv);
    for (int p = 0; p < 4; ++p) {
        // A W16^p = exp(-2 pi i (a / n + p / 16))
        const double e = a * 16.0 + p * n;   // over 16 n
        out[2 + 2 * p] = tan_pair(e, 16 * n, inv);
        out[3 + 2 * p] = tan_pair(2 * e, 16 * n, inv);
    }
}

std::vector<float2> dit4k_table()
{
    std::vector<float2> h(sc::DIT4K_TABLE_FLOAT2, make_float2(0.f, 0.f));
    item_pairs(&h[sc::DIT4K_P1B1], 1, 32, false);
    for (int var = 0; var < 3; ++var) {
        const bool inv = var == 2;
        for (int j = 0; j < 16; ++j)
            item_pairs(&h[sc::DIT4K_P2 + (var * 16 + j) * 10], var == 1 ? 2 * j + 1 : j,
                       var == 1 ? 512 : 256, inv);
        for (int j = 0; j < 256; ++j)
            item_pairs(&h[sc::DIT4K_P3 + (var * 256 + j) * 10], var == 1 ? 2 * j + 1 : j,
                       var == 1 ? 8192 : 4096, inv);
    }
    for (int k = 0; k < 4096; ++k) h[sc::DIT4K_UNP + k] = tan_pair(k, 8192, true);
    // The matrix-core first pass (bf16 storage): branch u's pass 1 is
    //   X[k2] = sum_q x[q] F(q, k2),  F = W_16^{q k2} (u = 0),  W_32^{q (2 k2 + 1)} (u = 1)
    // (branch 1's input rotation W_32^q merged), as a real 32 x 32 matrix: row 2 k2 + c
    // (c = 0 real, 1 imaginary part of X[k2]), column 2 q + d (d = 0 the real part v of
    // x[q], 1 the imaginary part g).  Each entry m is the sum of three bf16 parts
    // (hi = bf16(m), mid = bf16(m - hi), lo = bf16(m - hi - mid): within 2^-26 |m|).  A
    // 32 x 32 x 16 bf16 product's A fragment: lane l holds row l % 32 and the 8 columns
    // 16 h + 8 (l / 32) + e, e < 8, of K half h, column e in the low half of 32-bit word e/2.
    auto bf16_rne = [](double x) -> uint16_t {
        const float f = (float)x;
        uint32_t b;
        std::memcpy(&b, &f, 4);
        b += 0x7fffu + ((b >> 16) & 1u);
        return (uint16_t)(b >> 16);
    };
    auto bf16_val = [](uint16_t hb) -> double {
        const uint32_t b = (uint32_t)hb << 16;
        float f;
        std::memcpy(&f, &b, 4);
        return f;
    };
    for (int u = 0; u < 2; ++u)
        for (int kh = 0; kh < 2; ++kh)
            for (int lane = 0; lane < 64; ++lane) {
                uint16_t parts[3][8];
                for (int e = 0; e < 8; ++e) {
                    const int i = lane % 32, kk = 16 * kh + 8 * (lane / 32) + e;
                    const int k2 = i / 2, c = i % 2, q = kk / 2, dd = kk % 2;
                    // F = exp(-2 pi i a / 32): a = 2 q k2 (u = 0) or q (2 k2 + 1) (u = 1)
                    const double a = u == 0 ? 2.0 * q * k2 : (double)q * (2 * k2 + 1);
                    const double ang = 6.283185307179586476925286766559 * a / 32.0;
                    const double fr = std::cos(ang), fi = -std::sin(ang);
                    // out.re = fr x.re - fi x.im, out.im = fi x.re + fr x.im
                    const double m = c == 0 ? (dd == 0 ? fr : -fi) : (dd == 0 ? fi : fr);
                    const uint16_t p0 = bf16_rne(m);
                    const double r1 = m - bf16_val(p0);
                    const uint16_t p1 = bf16_rne(r1);
                    const uint16_t p2 = bf16_rne(r1 - bf16_val(p1));
                    parts[0][e] = p0;
                    parts[1][e] = p1;
                    parts[2][e] = p2;
                }
                for (int t = 0; t < 3; ++t) {
                    uint32_t w[4];
                    for (int j = 0; j < 4; ++j)
                        w[j] = (uint32_t)parts[t][2 * j] | ((uint32_t)parts[t][2 * j + 1] << 16);
                    float2* dst = &h[sc::DIT4K_MF + ((u * 3 + t) * 2 + kh) * 128 + 2 * lane];
                    std::memcpy(dst, w, 16);
                }
            }
    return h;
}

// the table of the M = 1024 or 2048 kernel (layout in sc_internal.h)
std::vector<float2> dit_table(int M)
{
    const int R1 = M / 256, TB = M / 16;
    std::vector<float2> h(sc::dit_table_size(M), make_float2(0.f, 0.f));
    if (R1 == 4) {
        h[sc::DIT_P1B1] = tan_pair(1, 8, false);
        h[sc::DIT_P1B1 + 1] = tan_pair(2, 8, false);
    } else {
        // T = W_16: T^2, T^4, then U_p = T W_8^p = W_16^{1 + 2p}
        h[sc::DIT_P1B1] = tan_pair(2, 16, false);
        h[sc::DIT_P1B1 + 1] = tan_pair(4, 16, false);
        for (int p = 0; p < 4; ++p) h[sc::DIT_P1B1 + 2 + p] = tan_pair(1 + 2 * p, 16, false);
    }
    for (int var = 0; var < 3; ++var) {
        const bool inv = var == 2;
        for (int j = 0; j < R1; ++j)
            item_pairs(&h[sc::dit_p2(M) + (var * R1 + j) * 10], var == 1 ? 2 * j + 1 : j,
                       var == 1 ? 32 * R1 : 16 * R1, inv);
        for (int j = 0; j < TB; ++j)
            item_pairs(&h[sc::dit_p3(M) + (var * TB + j) * 10], var == 1 ? 2 * j + 1 : j,
                       var == 1 ? 2 * M : M, inv);
    }
    for (int k = 0; k < M; ++k) h[sc::dit_unp(M) + k] = tan_pair(k, 2 * M, true);
    return h;
}

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

// exp(-2 pi i k / n) in float64, rounded once to float32; exact zeros and ones on the axes
float2 unit_root(int64_t k, int64_t n)
{
    k %= n;
    if (k < 0) k += n;
    if (4 * k == 0) return make_float2(1.f, 0.f);
    if (4 * k == n) return make_float2(0.f, -1.f);
    if (4 * k == 2 * n) return make_float2(-1.f, 0.f);
    if (4 * k == 3 * n) return make_float2(0.f, 1.f);
    const double a = 6.283185307179586476925286766559 * (double)k / (double)n;
    return make_float2((float)std::cos(a), (float)-std::sin(a));
}

// Building a table is a blocking upload, which a stream under graph capture must not see:
// with `stream` being captured, a missing table is SC_ERR_UNSUPPORTED (sc_prepare builds
// the tables beforehand).
sc_status capture_forbids_build(hipStream_t stream)
{
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return SC_ERR_HIP;
    return cap == hipStreamCaptureStatusNone ? SC_OK : SC_ERR_UNSUPPORTED;
}

sc_status device_state(DeviceState** out, bool need_ntt, hipStream_t stream,
                       bool may_build = true)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SC_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceState& d = g_dev[dev];
    if (!d.fused_tw || (need_ntt && !d.ntt_ready)) {
        if (!may_build) return SC_ERR_UNSUPPORTED;
        const sc_status cs = capture_forbids_build(stream);
        if (cs != SC_OK) return cs;
    }
    if (!d.fused_tw) {
        std::vector<float2> h(sc::FUSED_BANK_FLOAT2);
        for (int i = 0; i < sc::FUSED_TW_N; ++i) h[i] = unit_root(i, sc::FUSED_TW_N);
        for (int Q = 32; Q <= 4096; Q *= 2)
            for (int k = 0; k < 16; ++k)
                for (int n = 0; n < Q / 16; ++n)
                    h[sc::FUSED_TW_N + (Q - 32) + k * (Q / 16) + n] = unit_root((int64_t)n * k, Q);
        for (int Q = 16; Q <= 4096; Q *= 2)
            for (int k = 0; k < 8; ++k)
                for (int n = 0; n < Q / 8; ++n)
                    h[sc::FUSED_TW_N + (2 * 4096 - 32) + (Q - 16) + k * (Q / 8) + n] =
                        unit_root((int64_t)n * k, Q);
        void* p = nullptr;
        sc_status st = upload(h.data(), h.size() * sizeof(float2), &p);
        if (st != SC_OK) return st;
        const std::vector<float2> t4 = dit4k_table();
        void* p4 = nullptr;
        if ((st = upload(t4.data(), t4.size() * sizeof(float2), &p4)) != SC_OK) {
            (void)hipFree(p);
            return st;
        }
        void* pd[2] = {nullptr, nullptr};
        for (int i = 0; i < 2 && st == SC_OK; ++i) {
            const std::vector<float2> t = dit_table(1024 << i);
            st = upload(t.data(), t.size() * sizeof(float2), &pd[i]);
        }
        if (st != SC_OK) {
            if (pd[0]) (void)hipFree(pd[0]);
            (void)hipFree(p4);
            (void)hipFree(p);
            return st;
        }
        d.dit[0] = (float2*)pd[0];
        d.dit[1] = (float2*)pd[1];
        d.dit4k = (float2*)p4;
        d.fused_tw = (float2*)p;
    }
    if (need_ntt && !d.ntt_ready) {
        for (int k = 0; k < 3; ++k) {
            sc_status st = build_ntt_tables(&d.ntt[k], sc::NTT_PRIMES[k]);
            if (st != SC_OK) return st;
        }
        d.ntt_ready = true;
    }
    *out = &d;
    return SC_OK;
}

// four-step twiddle tables for one M (built once per device and M)
sc_status fourstep_tables(DeviceState& d, int M, sc::FsTw* out, hipStream_t stream,
                          bool may_build = true)
{
    auto it = d.fs.find(M);
    if (it != d.fs.end()) {
        *out = it->second;
        return SC_OK;
    }
    if (!may_build) return SC_ERR_UNSUPPORTED;
    const sc_status cs = capture_forbids_build(stream);
    if (cs != SC_OK) return cs;
    int M1, M2;
    sc::fourstep_split(M, &M1, &M2);
    const int64_t N = 2 * (int64_t)M, H = M2 / 2, U = M2 / 4 + 1;
    const size_t nn = (size_t)N, na = (size_t)M, nb = (size_t)M1 * H, nu = (size_t)2 * M1 * U;
    std::vector<float2> h(nn + na + nb + nu);
    float2* tn = h.data();
    float2* ta = tn + nn;
    float2* tb = ta + na;
    float2* tu = tb + nb;
    for (int64_t e = 0; e < N; ++e) tn[e] = unit_root(e, N);
    for (int64_t k2 = 0; k2 < M1; ++k2)
        for (int64_t n1 = 0; n1 < M2; ++n1) ta[k2 * M2 + n1] = unit_root(n1 * k2, M);
    for (int64_t i2 = 0; i2 < M1; ++i2)
        for (int64_t m1 = 0; m1 < H; ++m1) tb[i2 * H + m1] = unit_root(m1 * i2, M / 2);
    for (int64_t r2 = 0; r2 < 2 * M1; ++r2)
        for (int64_t k1 = 0; k1 < U; ++k1)
            tu[r2 * U + k1] = unit_root(2 * (M1 * k1 + (r2 >> 1)) + (r2 & 1), N);
    void* p = nullptr;
    sc_status st = upload(h.data(), h.size() * sizeof(float2), &p);
    if (st != SC_OK) return st;
    const float2* base = (const float2*)p;
    sc::FsTw t{base, base + nn, base + nn + na, base + nn + na + nb};
    d.fs[M] = t;
    *out = t;
    return SC_OK;
}

// the four-step NTT's tables for transform length M modulo NTT_PRIMES[prime] (as doubles,
// made on first use): w_N^j (N = 2M, j < N) and the column and row twiddles in lane order;
// under graph capture (or with may_build false) a missing table is SC_ERR_UNSUPPORTED.  Caller holds g_mu.
sc_status ntt4_table(DeviceState& d, int M, int prime, const double** out, hipStream_t stream,
                     bool may_build = true)
{
    auto it = d.ntt4.find({M, prime});
    if (it != d.ntt4.end()) {
        *out = it->second;
        return SC_OK;
    }
    if (!may_build) return SC_ERR_UNSUPPORTED;
    const sc_status cs = capture_forbids_build(stream);
    if (cs != SC_OK) return cs;
    const uint64_t p = sc::NTT_PRIMES[prime];
    const int64_t N = 2 * (int64_t)M;
    const uint64_t w = powmod(3, (p - 1) / (uint64_t)N, p);
    // w_N^j, j < N; then w_N^{n1 (2 k2 + b)} at [b][k2][n1]; then w_M^{-m1 k2} at [k2][m1]
    const int64_t M2 = 4096, M1 = M / M2;
    std::vector<uint64_t> pw((size_t)N);
    uint64_t x = 1;
    for (int64_t j = 0; j < N; ++j) {
        pw[j] = x;
        x = x * w % p;
    }
    std::vector<double> h((size_t)N + 2 * (size_t)M + (size_t)M);
    for (int64_t j = 0; j < N; ++j) h[j] = (double)pw[j];
    for (int64_t b = 0; b < 2; ++b)
        for (int64_t k2 = 0; k2 < M1; ++k2)
            for (int64_t n1 = 0; n1 < M2; ++n1)
                h[N + (b * M1 + k2) * M2 + n1] = (double)pw[(n1 * (2 * k2 + b)) % N];
    for (int64_t k2 = 0; k2 < M1; ++k2)
        for (int64_t m1 = 0; m1 < M2; ++m1)
            h[2 * N + k2 * M2 + m1] = (double)pw[(2 * (M - (m1 * k2) % M)) % N];
    void* dp = nullptr;
    const sc_status st = upload(h.data(), h.size() * sizeof(double), &dp);
    if (st != SC_OK) return st;
    d.ntt4[{M, prime}] = (const double*)dp;
    *out = (const double*)dp;
    return SC_OK;
}

size_t elt_size(sc_kind k) { return k == SC_KIND_BF16 ? 2 : 4; }

int64_t next_pow2(int64_t x)
{
    int64_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

bool overlaps(const void* a, const void* b, uint64_t bytes)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bytes && y < x + bytes;
}

// [a, a + na) and [b, b + nb) share a byte
bool ranges_overlap(const void* a, uint64_t na, const void* b, uint64_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

bool exact_kind(sc_kind k) { return k == SC_KIND_NTT_I32 || k == SC_KIND_FIXED_F32; }

// Kind and shape checks.  *n receives B*C*L.
sc_status check_shape(sc_kind kind, int64_t B, int64_t C, int64_t L, int64_t* n)
{
    if (kind != SC_KIND_F32 && kind != SC_KIND_BF16 && kind != SC_KIND_NTT_I32 &&
        kind != SC_KIND_FIXED_F32)
        return SC_ERR_INVALID_ARGUMENT;
    if (B < 0 || C < 0 || L < 0) return SC_ERR_INVALID_ARGUMENT;
    const __int128 total = (__int128)B * (__int128)C * (__int128)L;
    if (total * (__int128)elt_size(kind) > (__int128)INT64_MAX) return SC_ERR_INVALID_ARGUMENT;
    *n = (int64_t)total;
    return SC_OK;
}

// Host-side checks common to every entry point.  *n receives B*C*L.
sc_status check_args(sc_kind kind, const void* v, const void* g, const void* r, int64_t B,
                     int64_t C, int64_t L, int64_t* n)
{
    const sc_status st = check_shape(kind, B, C, L, n);
    if (st != SC_OK) return st;
    const size_t es = elt_size(kind);
    const int64_t total = *n;
    if (total == 0) return SC_OK;
    if (!v || !g || !r) return SC_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)v | (uintptr_t)g | (uintptr_t)r) % es) return SC_ERR_INVALID_ARGUMENT;
    const uint64_t bytes = (uint64_t)total * es;
    if (overlaps(r, v, bytes) || overlaps(r, g, bytes)) return SC_ERR_INVALID_ARGUMENT;
    return SC_OK;
}

sc_status resolve_path(sc_kind kind, int64_t L, int32_t requested, sc_path* out)
{
    const bool fl = !exact_kind(kind);
    switch (requested) {
    case SC_PATH_AUTO:
        if (!fl) {
            if (L <= kMaxLNtt) *out = SC_PATH_FUSED;
            else if (L <= sc::NTT4_MAX_L) *out = SC_PATH_FOUR_STEP;
            else return SC_ERR_UNSUPPORTED;
        } else if (L <= sc::DIRECT_MAX_L) {
            *out = SC_PATH_DIRECT;
        } else if (L <= kMaxLFused) {
            *out = SC_PATH_FUSED;
        } else if (L <= sc::FOURSTEP_MAX_L) {
            *out = SC_PATH_FOUR_STEP;
        } else {
            return SC_ERR_UNSUPPORTED;
        }
        return SC_OK;
    case SC_PATH_FUSED:
        if (L > (fl ? kMaxLFused : kMaxLNtt)) return SC_ERR_UNSUPPORTED;
        *out = SC_PATH_FUSED;
        return SC_OK;
    case SC_PATH_DIRECT:
        if (!fl || L > kMaxLFused) return SC_ERR_UNSUPPORTED;
        *out = SC_PATH_DIRECT;
        return SC_OK;
    case SC_PATH_FOUR_STEP:
        if (!fl) {
            // the exact kind's four-step split has rows of 4096: L above the fused range only
            if (L <= kMaxLNtt || L > sc::NTT4_MAX_L) return SC_ERR_UNSUPPORTED;
            *out = SC_PATH_FOUR_STEP;
            return SC_OK;
        }
        if (L < kMinLFourStep || L > sc::FOURSTEP_MAX_L) return SC_ERR_UNSUPPORTED;
        *out = SC_PATH_FOUR_STEP;
        return SC_OK;
    case SC_PATH_NTT_MFMA:
        if (kind != SC_KIND_NTT_I32 || L > kMaxLNtt) return SC_ERR_UNSUPPORTED;
        *out = SC_PATH_NTT_MFMA;
        return SC_OK;
    case SC_PATH_FUSED_MFMA:
        // the M = 4096 kernel's matrix-core first pass (bf16 storage)
        if (kind != SC_KIND_BF16 || L <= 2048 || L > 4096 || !kFused4k)
            return SC_ERR_UNSUPPORTED;
        *out = SC_PATH_FUSED_MFMA;
        return SC_OK;
    default:
        return SC_ERR_INVALID_ARGUMENT;
    }
}

// the four-step path's second stream and events of the current device, made on first use
sc_status fourstep_streams(DeviceState& d)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (d.fs_side) return SC_OK;
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return SC_ERR_HIP;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
        if (f) (void)hipEventDestroy(f);
        (void)hipStreamDestroy(s);
        return SC_ERR_HIP;
    }
    d.fs_fork = f;
    d.fs_join = j;
    d.fs_side = s;
    return SC_OK;
}

// four-step scratch: channels per chunk and bytes needed
// scratch bytes per channel of the four-step path of this kind
size_t fourstep_per_channel(sc_kind kind, int64_t L)
{
    const int M = (int)next_pow2(L);
    return kind == SC_KIND_NTT_I32     ? sc::ntt4_bytes_per_channel(M)
           : kind == SC_KIND_FIXED_F32 ? sc::fixed4_bytes_per_channel(M)
                                       : sc::fourstep_bytes_per_channel(M);
}

void fourstep_plan(sc_kind kind, int64_t nch, int64_t L, int64_t* chunk, size_t* bytes,
                   int64_t budget = kFourStepChunkBytes)
{
    const int64_t per = (int64_t)fourstep_per_channel(kind, L);
    int64_t c = budget / per;
    if (c < 1) c = 1;
    if (c > nch) c = nch;
    // exact kinds: the fewest chunks the budget allows, of balanced sizes (no short last
    // chunk); the float kinds' chunks are run as two halves on two streams
    if (exact_kind(kind) && c > 0) {
        const int64_t k = (nch + c - 1) / c;
        c = (nch + k - 1) / k;
    }
    *chunk = c;
    *bytes = (size_t)(c * per);
}

// Whether a four-step call runs its parts on two streams (then made here, once per device):
// not when there is a single part, when the caller's stream is being captured into a graph,
// or when the call may not create the second stream (allocation-free entry point).
sc_status use_second_stream(DeviceState& d, hipStream_t stream, bool noalloc, int64_t nch,
                            int64_t chunk, bool* two)
{
    *two = false;
    if (noalloc || chunk < 2 || nch <= chunk / 2) return SC_OK;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return SC_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return SC_OK;
    const sc_status st = fourstep_streams(d);
    if (st == SC_OK) *two = true;
    return st;
}

// One convolution of a call: o = causal(a, b) per channel, or with rev the gradient form
// o = rev(causal(rev(a), b)).
struct Job {
    const void* a;
    const void* b;
    void* o;
};

// Runs the jobs of one call (arguments already checked) on one path with one scratch area,
// which the jobs use one after the other in stream order.
// With noalloc (the allocation-free entry point): ws is the static scratch of ws_bytes,
// four-step chunks are sized to it (a channel that does not fit is SC_ERR_UNSUPPORTED), the
// call stays on `stream`, and a missing table is SC_ERR_UNSUPPORTED instead of being built.
sc_status run_jobs(sc_kind kind, const Job* jobs, int njobs, bool rev, int64_t n, int64_t B,
                   int64_t C, int64_t L, const sc_options* opt, void* ws, size_t ws_bytes,
                   hipStream_t stream, bool noalloc = false)
{
    int32_t req = SC_PATH_AUTO, head = kDefaultHead, fv = 0, fg = 0;
    if (opt) {
        for (int i = 0; i < 4; ++i)
            if (opt->reserved[i]) return SC_ERR_INVALID_ARGUMENT;
        req = opt->path;
        if (opt->head != -1) {
            if (opt->head < 0 || opt->head > kMaxHead) return SC_ERR_INVALID_ARGUMENT;
            head = (opt->head + 1) & ~1;
        }
        fv = opt->frac_v;
        fg = opt->frac_g;
        if (kind != SC_KIND_FIXED_F32 && (fv || fg)) return SC_ERR_INVALID_ARGUMENT;
        if (fv < -kMaxFrac || fv > kMaxFrac || fg < -kMaxFrac || fg > kMaxFrac)
            return SC_ERR_INVALID_ARGUMENT;
    }
    if (kind == SC_KIND_FIXED_F32 && rev) return SC_ERR_UNSUPPORTED;
    sc_path path;
    sc_status st = resolve_path(kind, L, req, &path);
    if (st != SC_OK) return st;
    if (n == 0) return SC_OK;
    const int64_t nch = B * C;

    // scratch of this path, checked against a caller workspace before any HIP call
    size_t need = 0;
    int64_t chunk = 0;
    if (path == SC_PATH_FOUR_STEP) {
        if (noalloc && fourstep_per_channel(kind, L) > (size_t)ws_bytes)
            return SC_ERR_UNSUPPORTED;
        fourstep_plan(kind, nch, L, &chunk, &need,
                      noalloc ? (int64_t)ws_bytes : kFourStepChunkBytes);
    }
    if (need > 0) {
        if (ws) {
            if (ws_bytes < need) return SC_ERR_WORKSPACE;
            if ((uintptr_t)ws % 256) return SC_ERR_INVALID_ARGUMENT;
        } else if (ws_bytes) {
            return SC_ERR_INVALID_ARGUMENT;
        }
    }

    DeviceState* d = nullptr;
    st = device_state(&d, exact_kind(kind), stream, !noalloc);
    if (st != SC_OK) return st;

    hipError_t e = hipSuccess;
    if (exact_kind(kind) && path == SC_PATH_FOUR_STEP) {
        const int M = (int)next_pow2(L);
        const bool fix = kind == SC_KIND_FIXED_F32;
        const double* wtab[3] = {nullptr, nullptr, nullptr};
        {
            std::lock_guard<std::mutex> lk(g_mu);
            for (int i = 0; i < (fix ? 3 : 1) && st == SC_OK; ++i)
                st = ntt4_table(*d, M, i, &wtab[i], stream, !noalloc);
        }
        if (st != SC_OK) return st;
        // two streams take alternate halves of the chunks, as on the float path (one part's
        // column kernels overlap the other's row kernel), under the same conditions
        bool two = false;
        if ((st = use_second_stream(*d, stream, noalloc, nch, chunk, &two)) != SC_OK) return st;
        std::unique_lock<std::mutex> order(d->fs_mu, std::defer_lock);
        if (two) order.lock();
        void* scratch = ws;
        bool own = false;
        if (!ws) {
            if (hipMallocAsync(&scratch, need, stream) != hipSuccess) return SC_ERR_HIP;
            own = true;
        }
        hipStream_t side = two ? d->fs_side : nullptr;
        hipEvent_t fork = two ? d->fs_fork : nullptr, join = two ? d->fs_join : nullptr;
        for (int k = 0; k < njobs && e == hipSuccess; ++k)
            e = fix ? sc::launch_fixed4((const float*)jobs[k].a, (const float*)jobs[k].b,
                                        (float*)jobs[k].o, nch, (int)L, M, fv, fg, d->ntt, wtab,
                                        scratch, need, chunk, stream, side, fork, join)
                    : sc::launch_ntt4((const int32_t*)jobs[k].a, (const int32_t*)jobs[k].b,
                                      (int32_t*)jobs[k].o, nch, (int)L, M, rev, d->ntt[0],
                                      wtab[0], scratch, need, chunk, stream, side, fork, join);
        if (own && hipFreeAsync(scratch, stream) != hipSuccess && e == hipSuccess)
            e = hipErrorUnknown;
        return e == hipSuccess ? SC_OK : SC_ERR_HIP;
    }
    if (kind == SC_KIND_FIXED_F32) {
        const int M = (int)std::max<int64_t>(64, next_pow2(L));
        for (int k = 0; k < njobs && e == hipSuccess; ++k)
            e = sc::launch_fixed((const float*)jobs[k].a, (const float*)jobs[k].b,
                                 (float*)jobs[k].o, nch, (int)L, M, fv, fg, d->ntt, stream);
        return e == hipSuccess ? SC_OK : SC_ERR_HIP;
    }
    if (kind == SC_KIND_NTT_I32 && path == SC_PATH_NTT_MFMA) {
        {
            std::lock_guard<std::mutex> lk(g_mu);
            if (!d->mfma_ready) {
                if (noalloc) return SC_ERR_UNSUPPORTED;
                if ((st = capture_forbids_build(stream)) != SC_OK) return st;
                if ((st = build_mfma_tables(&d->mfma)) != SC_OK) return st;
                d->mfma_ready = true;
            }
        }
        const int M = (int)std::max<int64_t>(64, next_pow2(L));
        for (int k = 0; k < njobs && e == hipSuccess; ++k)
            e = sc::launch_ntt_mfma((const int32_t*)jobs[k].a, (const int32_t*)jobs[k].b,
                                    (int32_t*)jobs[k].o, nch, (int)L, M, rev, d->mfma, stream);
        return e == hipSuccess ? SC_OK : SC_ERR_HIP;
    }
    if (kind == SC_KIND_NTT_I32) {
        const int M = (int)std::max<int64_t>(64, next_pow2(L));
        for (int k = 0; k < njobs && e == hipSuccess; ++k)
            e = sc::launch_ntt((const int32_t*)jobs[k].a, (const int32_t*)jobs[k].b,
                               (int32_t*)jobs[k].o, nch, (int)L, M, rev, d->ntt[0], stream);
        return e == hipSuccess ? SC_OK : SC_ERR_HIP;
    }
    const sc::Store s = kind == SC_KIND_F32 ? sc::Store::F32 : sc::Store::BF16;
    bool pair = L % 2 == 0;
    for (int k = 0; k < njobs; ++k)
        pair = pair && (uintptr_t)jobs[k].o % (2 * elt_size(kind)) == 0;
    if (path == SC_PATH_DIRECT) {
        for (int k = 0; k < njobs && e == hipSuccess; ++k)
            e = sc::launch_direct(s, jobs[k].a, jobs[k].b, jobs[k].o, nch, (int)L, rev, stream);
    } else if (path == SC_PATH_FUSED_MFMA) {
        for (int k = 0; k < njobs && e == hipSuccess; ++k)
            e = sc::launch_fused4k(s, jobs[k].a, jobs[k].b, jobs[k].o, nch, (int)L, head, pair,
                                   rev, true, d->dit4k, stream);
    } else if (path == SC_PATH_FUSED) {
        const int M = (int)std::max<int64_t>(64, next_pow2(L));
        for (int k = 0; k < njobs && e == hipSuccess; ++k)
            e = M == 4096 && kFused4k
                    ? sc::launch_fused4k(s, jobs[k].a, jobs[k].b, jobs[k].o, nch, (int)L, head,
                                         pair, rev, false, d->dit4k, stream)
                : (M == 1024 || M == 2048) && kFusedDit
                    ? sc::launch_fused_dit(s, jobs[k].a, jobs[k].b, jobs[k].o, nch, (int)L, M,
                                           head, pair, rev, d->dit[M == 2048], stream)
                    : sc::launch_fused(s, jobs[k].a, jobs[k].b, jobs[k].o, nch, (int)L, M, head,
                                       pair, rev, d->fused_tw, stream);
    } else {
        const int M = (int)next_pow2(L);
        sc::FsTw tw;
        {
            std::lock_guard<std::mutex> lk(g_mu);
            st = fourstep_tables(*d, M, &tw, stream, !noalloc);
        }
        if (st != SC_OK) return st;
        // two streams take alternate halves of the chunks (measured 1.54 -> 1.34 ms on the
        // long workload: one part's memory-bound column kernels overlap the other's rows)
        bool two = false;
        if ((st = use_second_stream(*d, stream, noalloc, nch, chunk, &two)) != SC_OK) return st;
        std::unique_lock<std::mutex> order(d->fs_mu, std::defer_lock);
        if (two) order.lock();
        void* scratch = ws;
        bool own = false;
        if (!ws) {
            if (hipMallocAsync(&scratch, need, stream) != hipSuccess) return SC_ERR_HIP;
            own = true;
        }
        for (int k = 0; k < njobs && e == hipSuccess; ++k)
            e = sc::launch_fourstep(s, jobs[k].a, jobs[k].b, jobs[k].o, nch, (int)L, M, head, pair,
                                    rev, d->fused_tw, tw, scratch, need, chunk, stream,
                                    two ? d->fs_side : nullptr, two ? d->fs_fork : nullptr,
                                    two ? d->fs_join : nullptr);
        if (own && hipFreeAsync(scratch, stream) != hipSuccess && e == hipSuccess)
            e = hipErrorUnknown;
    }
    return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

sc_status run(sc_kind kind, const void* v, const void* g, void* r, int64_t B, int64_t C,
              int64_t L, const sc_options* opt, void* ws, size_t ws_bytes, hipStream_t stream)
{
    int64_t n = 0;
    const sc_status st = check_args(kind, v, g, r, B, C, L, &n);
    if (st != SC_OK) return st;
    const Job job{v, g, r};
    return run_jobs(kind, &job, 1, false, n, B, C, L, opt, ws, ws_bytes, stream);
}

// Gradients: dv = rev(causal(rev(dr), g)), dg = rev(causal(rev(dr), v)).
sc_status run_bwd(sc_kind kind, const void* dr, const void* v, const void* g, void* dv, void* dg,
                  int64_t B, int64_t C, int64_t L, const sc_options* opt, void* ws,
                  size_t ws_bytes, hipStream_t stream)
{
    int64_t n = 0;
    sc_status st = check_shape(kind, B, C, L, &n);
    if (st != SC_OK) return st;
    if (n > 0) {
        if (!dr || !v || !g || !dv || !dg) return SC_ERR_INVALID_ARGUMENT;
        const size_t es = elt_size(kind);
        if (((uintptr_t)dr | (uintptr_t)v | (uintptr_t)g | (uintptr_t)dv | (uintptr_t)dg) % es)
            return SC_ERR_INVALID_ARGUMENT;
        const uint64_t bytes = (uint64_t)n * es;
        for (const void* out : {(const void*)dv, (const void*)dg})
            for (const void* in : {dr, v, g})
                if (overlaps(out, in, bytes)) return SC_ERR_INVALID_ARGUMENT;
        if (overlaps(dv, dg, bytes)) return SC_ERR_INVALID_ARGUMENT;
    }
    const Job jobs[2] = {{dr, g, dv}, {dr, v, dg}};
    return run_jobs(kind, jobs, 2, true, n, B, C, L, opt, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- staged calls

// Staging budget of the token-major and gate calls: the staged buffers of one chunk (v, g, r,
// or g alone) share about this many bytes, well inside the 256 MB last-level cache.
constexpr int64_t kStageBudget = (int64_t)96 << 20;
constexpr int64_t kGateGroup = 64;   // channels per gate group (one head)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BlcPlan {
    int64_t nb, cw;   // batch rows and channels per chunk
    size_t stage;     // bytes of one staged buffer
    size_t inner;     // scratch of the convolution path for one chunk
    size_t total;
};

// Chunks of whole batch rows when one row's C L elements fit a buffer, else blocks of 64k
// channels of one row (64k also keeps gate groups whole).
sc_status blc_plan(sc_kind kind, int64_t B, int64_t L, int64_t C, const sc_options* opt,
                   int nstage, BlcPlan* p)
{
    const int64_t elems = kStageBudget / nstage / (int64_t)elt_size(kind);   // per buffer
    if (C * L <= elems) {
        p->cw = C;
        p->nb = std::min<int64_t>(B, std::max<int64_t>(1, elems / (C * L)));
    } else {
        p->nb = 1;
        p->cw = std::min<int64_t>(C, std::max<int64_t>(64, elems / L / 64 * 64));
    }
    const int64_t nch = p->nb * p->cw;
    p->stage = align256((size_t)(nch * L) * elt_size(kind));
    sc_path path;
    const sc_status st = resolve_path(kind, L, opt ? opt->path : SC_PATH_AUTO, &path);
    if (st != SC_OK) return st;
    p->inner = 0;
    if (path == SC_PATH_FOUR_STEP) {
        int64_t chunk;
        fourstep_plan(kind, nch, L, &chunk, &p->inner);
    }
    p->total = (size_t)nstage * p->stage + align256(p->inner);
    return SC_OK;
}

// Staged calls, chunk by chunk through a workspace:
//  * token-major (tm) without gate: v, g, r in (B, L, C); transpose v and g into channel
//    rows, convolve, transpose the result back;
//  * token-major with gate (W not null; s takes g's place): transpose v, make g from s by
//    the gate kernel straight into channel rows, convolve, transpose back;
//  * channel-major with gate: g of the chunk from s into the workspace, convolve v with it
//    into r in place.
sc_status staged_run(sc_kind kind, bool tm, const void* v, const void* g, const void* W,
                     void* r, int64_t B, int64_t L, int64_t C, const sc_options* opt, void* ws,
                     size_t ws_bytes, hipStream_t stream)
{
    const bool gate = W != nullptr;
    int64_t n = 0;
    sc_status st = check_args(kind, v, g, r, B, C, L, &n);
    if (st != SC_OK) return st;
    const size_t es = elt_size(kind);
    if (gate) {
        if (kind != SC_KIND_F32 && kind != SC_KIND_BF16) return SC_ERR_INVALID_ARGUMENT;
        if (C % kGateGroup || C > INT32_MAX) return SC_ERR_UNSUPPORTED;
        if (n > 0) {
            if ((uintptr_t)W % 16) return SC_ERR_INVALID_ARGUMENT;
            if (tm && (uintptr_t)g % 16) return SC_ERR_INVALID_ARGUMENT;
            if (ranges_overlap(r, (uint64_t)n * es, W, (uint64_t)C * kGateGroup * 3 * es))
                return SC_ERR_INVALID_ARGUMENT;
        }
    }
    sc_path path;
    st = resolve_path(kind, L, opt ? opt->path : SC_PATH_AUTO, &path);
    if (st != SC_OK) return st;
    if (n == 0) return SC_OK;
    BlcPlan p;
    st = blc_plan(kind, B, L, C, opt, tm ? 3 : 1, &p);
    if (st != SC_OK) return st;
    if (ws) {
        if (ws_bytes < p.total) return SC_ERR_WORKSPACE;
        if ((uintptr_t)ws % 256) return SC_ERR_INVALID_ARGUMENT;
        const uintptr_t w0 = (uintptr_t)ws, w1 = w0 + p.total, nbytes = (uintptr_t)n * es;
        for (const void* t : {v, g, (const void*)r})
            if ((uintptr_t)t < w1 && w0 < (uintptr_t)t + nbytes) return SC_ERR_INVALID_ARGUMENT;
        if (gate && ranges_overlap(ws, p.total, W, (uint64_t)C * kGateGroup * 3 * es))
            return SC_ERR_INVALID_ARGUMENT;
    } else if (ws_bytes) {
        return SC_ERR_INVALID_ARGUMENT;
    }
    DeviceState* d = nullptr;
    st = device_state(&d, exact_kind(kind), stream);
    if (st != SC_OK) return st;
    void* base = ws;
    bool own = false;
    if (!ws) {
        if (hipMallocAsync(&base, p.total, stream) != hipSuccess) return SC_ERR_HIP;
        own = true;
    }
    const sc::Store sk = kind == SC_KIND_F32 ? sc::Store::F32 : sc::Store::BF16;
    char* wg = (char*)base;                       // g of the chunk
    char* wv = tm ? wg + p.stage : nullptr;       // v of the chunk (token-major)
    char* wr = tm ? wv + p.stage : nullptr;       // r of the chunk (token-major)
    void* inner = p.inner ? (void*)((char*)base + (tm ? 3 : 1) * p.stage) : nullptr;
    for (int64_t b0 = 0; b0 < B && st == SC_OK; b0 += p.nb) {
        const int64_t nb = std::min(p.nb, B - b0);
        for (int64_t c0 = 0; c0 < C && st == SC_OK; c0 += p.cw) {
            const int64_t cw = std::min(p.cw, C - c0);
            const int64_t off = (tm ? b0 * L * C + c0 : (b0 * C + c0) * L) * (int64_t)es;
            hipError_t e = hipSuccess;
            if (tm)
                e = sc::launch_transpose((int)es, (const char*)v + off, wv,
                                         gate ? nullptr : (const char*)g + off, gate ? nullptr : wg,
                                         L, cw, C, L, L * C, cw * L, nb, false, stream);
            if (e == hipSuccess && gate)
                e = sc::launch_gate(sk, tm, (const char*)g + off,
                                    (const char*)W + c0 * kGateGroup * 3 * (int64_t)es, wg, nb, C,
                                    cw, L, cw, stream);
            if (e != hipSuccess) {
                st = SC_ERR_HIP;
                break;
            }
            const Job job{tm ? (const void*)wv : (const char*)v + off, wg,
                          tm ? (void*)wr : (char*)r + off};
            st = run_jobs(kind, &job, 1, false, nb * cw * L, nb, cw, L, opt, inner,
                          inner ? p.inner : 0, stream);
            if (st != SC_OK) break;
            if (tm && sc::launch_transpose((int)es, wr, (char*)r + off, nullptr, nullptr, cw, L, L,
                                           C, cw * L, L * C, nb, true, stream) != hipSuccess)
                st = SC_ERR_HIP;
        }
    }
    if (own && hipFreeAsync(base, stream) != hipSuccess && st == SC_OK) st = SC_ERR_HIP;
    return st;
}

sc_status blc_run(sc_kind kind, const void* v, const void* g, void* r, int64_t B, int64_t L,
                  int64_t C, const sc_options* opt, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return staged_run(kind, true, v, g, nullptr, r, B, L, C, opt, ws, ws_bytes, stream);
}

size_t staged_bytes(sc_kind kind, bool tm, bool gate, int64_t B, int64_t L, int64_t C)
{
    int64_t n = 0;
    if (check_shape(kind, B, C, L, &n) != SC_OK || n == 0) return 0;
    if (gate && ((kind != SC_KIND_F32 && kind != SC_KIND_BF16) || C % kGateGroup)) return 0;
    BlcPlan p;
    if (blc_plan(kind, B, L, C, nullptr, tm ? 3 : 1, &p) != SC_OK) return 0;
    return p.total;
}

// g = gate(s, W), channel-major, written directly
sc_status gate_run(sc_kind kind, const void* s, const void* W, void* g, int64_t B, int64_t C,
                   int64_t L, hipStream_t stream)
{
    int64_t n = 0;
    sc_status st = check_shape(kind, B, C, L, &n);
    if (st != SC_OK) return st;
    if (kind != SC_KIND_F32 && kind != SC_KIND_BF16) return SC_ERR_INVALID_ARGUMENT;
    if (C % kGateGroup || C > INT32_MAX || L > INT32_MAX) return SC_ERR_UNSUPPORTED;
    if (n == 0) return SC_OK;
    if (!s || !W || !g) return SC_ERR_INVALID_ARGUMENT;
    const size_t es = elt_size(kind);
    if (((uintptr_t)s | (uintptr_t)g) % es || (uintptr_t)W % 16) return SC_ERR_INVALID_ARGUMENT;
    const uint64_t nbytes = (uint64_t)n * es, wbytes = (uint64_t)C * kGateGroup * 3 * es;
    if (overlaps(g, s, nbytes) || ranges_overlap(g, nbytes, W, wbytes))
        return SC_ERR_INVALID_ARGUMENT;
    DeviceState* d = nullptr;
    st = device_state(&d, false, stream);
    if (st != SC_OK) return st;
    const sc::Store sk = kind == SC_KIND_F32 ? sc::Store::F32 : sc::Store::BF16;
    return sc::launch_gate(sk, false, s, W, g, B, C, C, L, C, stream) == hipSuccess ? SC_OK
                                                                                    : SC_ERR_HIP;
}

template <class F>
sc_status guarded(F&& f)
{
    try {
        return f();
    } catch (...) {
        return SC_ERR_HIP;
    }
}

}  // namespace

extern "C" {

sc_status sc_causal_conv_f32(const float* v, const float* g, float* r, int64_t B, int64_t C,
                             int64_t L, hipStream_t stream)
{
    return guarded([&] { return run(SC_KIND_F32, v, g, r, B, C, L, nullptr, nullptr, 0, stream); });
}

sc_status sc_causal_conv_bf16(const uint16_t* v, const uint16_t* g, uint16_t* r, int64_t B,
                              int64_t C, int64_t L, hipStream_t stream)
{
    return guarded([&] { return run(SC_KIND_BF16, v, g, r, B, C, L, nullptr, nullptr, 0, stream); });
}

sc_status sc_causal_conv_ntt_i32(const int32_t* v, const int32_t* g, int32_t* r, int64_t B,
                                 int64_t C, int64_t L, hipStream_t stream)
{
    return guarded(
        [&] { return run(SC_KIND_NTT_I32, v, g, r, B, C, L, nullptr, nullptr, 0, stream); });
}

size_t sc_workspace_bytes(sc_kind kind, int64_t B, int64_t C, int64_t L)
{
    try {
        int64_t n = 0;
        if (check_shape(kind, B, C, L, &n) != SC_OK || n == 0) return 0;
        sc_path path;
        if (resolve_path(kind, L, SC_PATH_AUTO, &path) != SC_OK) return 0;
        if (path != SC_PATH_FOUR_STEP) return 0;
        int64_t chunk;
        size_t need;
        fourstep_plan(kind, B * C, L, &chunk, &need);
        return need;
    } catch (...) {
        return 0;
    }
}

size_t sc_blc_workspace_bytes(sc_kind kind, int64_t B, int64_t L, int64_t C)
{
    try {
        return staged_bytes(kind, true, false, B, L, C);
    } catch (...) {
        return 0;
    }
}

sc_status sc_gate_f32(const float* s, const float* W, float* g, int64_t B, int64_t C, int64_t L,
                      hipStream_t stream)
{
    return guarded([&] { return gate_run(SC_KIND_F32, s, W, g, B, C, L, stream); });
}

sc_status sc_gate_bf16(const uint16_t* s, const uint16_t* W, uint16_t* g, int64_t B, int64_t C,
                       int64_t L, hipStream_t stream)
{
    return guarded([&] { return gate_run(SC_KIND_BF16, s, W, g, B, C, L, stream); });
}

size_t sc_gate_conv_workspace_bytes(sc_kind kind, int64_t B, int64_t C, int64_t L)
{
    try {
        return staged_bytes(kind, false, true, B, L, C);
    } catch (...) {
        return 0;
    }
}

size_t sc_gate_conv_blc_workspace_bytes(sc_kind kind, int64_t B, int64_t L, int64_t C)
{
    try {
        return staged_bytes(kind, true, true, B, L, C);
    } catch (...) {
        return 0;
    }
}

sc_status sc_gate_conv_ex(sc_kind kind, const void* v, const void* s, const void* W, void* r,
                          int64_t B, int64_t C, int64_t L, const sc_options* opt, void* ws,
                          size_t ws_bytes, hipStream_t stream)
{
    return guarded([&] {
        if (!W && B != 0 && C != 0 && L != 0) return SC_ERR_INVALID_ARGUMENT;
        return staged_run(kind, false, v, s, W ? W : (const void*)1, r, B, L, C, opt, ws, ws_bytes,
                          stream);
    });
}

sc_status sc_gate_conv_blc_ex(sc_kind kind, const void* v, const void* s, const void* W, void* r,
                              int64_t B, int64_t L, int64_t C, const sc_options* opt, void* ws,
                              size_t ws_bytes, hipStream_t stream)
{
    return guarded([&] {
        if (!W && B != 0 && C != 0 && L != 0) return SC_ERR_INVALID_ARGUMENT;
        return staged_run(kind, true, v, s, W ? W : (const void*)1, r, B, L, C, opt, ws, ws_bytes,
                          stream);
    });
}

sc_status sc_gate_conv_blc_f32(const float* v, const float* s, const float* W, float* r,
                               int64_t B, int64_t L, int64_t C, hipStream_t stream)
{
    return sc_gate_conv_blc_ex(SC_KIND_F32, v, s, W, r, B, L, C, nullptr, nullptr, 0, stream);
}

sc_status sc_gate_conv_blc_bf16(const uint16_t* v, const uint16_t* s, const uint16_t* W,
                                uint16_t* r, int64_t B, int64_t L, int64_t C, hipStream_t stream)
{
    return sc_gate_conv_blc_ex(SC_KIND_BF16, v, s, W, r, B, L, C, nullptr, nullptr, 0, stream);
}

sc_status sc_causal_conv_blc_f32(const float* v, const float* g, float* r, int64_t B, int64_t L,
                                 int64_t C, hipStream_t stream)
{
    return guarded([&] { return blc_run(SC_KIND_F32, v, g, r, B, L, C, nullptr, nullptr, 0, stream); });
}

sc_status sc_causal_conv_blc_bf16(const uint16_t* v, const uint16_t* g, uint16_t* r, int64_t B,
                                  int64_t L, int64_t C, hipStream_t stream)
{
    return guarded([&] { return blc_run(SC_KIND_BF16, v, g, r, B, L, C, nullptr, nullptr, 0, stream); });
}

sc_status sc_causal_conv_blc_ex(sc_kind kind, const void* v, const void* g, void* r, int64_t B,
                                int64_t L, int64_t C, const sc_options* opt, void* ws,
                                size_t ws_bytes, hipStream_t stream)
{
    return guarded([&] { return blc_run(kind, v, g, r, B, L, C, opt, ws, ws_bytes, stream); });
}

sc_status sc_causal_conv_f32_ws(const float* v, const float* g, float* r, int64_t B, int64_t C,
                                int64_t L, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return guarded([&] { return run(SC_KIND_F32, v, g, r, B, C, L, nullptr, ws, ws_bytes, stream); });
}

sc_status sc_causal_conv_bf16_ws(const uint16_t* v, const uint16_t* g, uint16_t* r, int64_t B,
                                 int64_t C, int64_t L, void* ws, size_t ws_bytes,
                                 hipStream_t stream)
{
    return guarded([&] { return run(SC_KIND_BF16, v, g, r, B, C, L, nullptr, ws, ws_bytes, stream); });
}

sc_status sc_causal_conv_ntt_i32_ws(const int32_t* v, const int32_t* g, int32_t* r, int64_t B,
                                    int64_t C, int64_t L, void* ws, size_t ws_bytes,
                                    hipStream_t stream)
{
    return guarded(
        [&] { return run(SC_KIND_NTT_I32, v, g, r, B, C, L, nullptr, ws, ws_bytes, stream); });
}

sc_status sc_causal_conv_ex(sc_kind kind, const void* v, const void* g, void* r, int64_t B,
                            int64_t C, int64_t L, const sc_options* opt, void* ws,
                            size_t ws_bytes, hipStream_t stream)
{
    return guarded([&] { return run(kind, v, g, r, B, C, L, opt, ws, ws_bytes, stream); });
}

sc_status sc_causal_conv_bwd_f32(const float* dr, const float* v, const float* g, float* dv,
                                 float* dg, int64_t B, int64_t C, int64_t L, hipStream_t stream)
{
    return guarded([&] {
        return run_bwd(SC_KIND_F32, dr, v, g, dv, dg, B, C, L, nullptr, nullptr, 0, stream);
    });
}

sc_status sc_causal_conv_bwd_bf16(const uint16_t* dr, const uint16_t* v, const uint16_t* g,
                                  uint16_t* dv, uint16_t* dg, int64_t B, int64_t C, int64_t L,
                                  hipStream_t stream)
{
    return guarded([&] {
        return run_bwd(SC_KIND_BF16, dr, v, g, dv, dg, B, C, L, nullptr, nullptr, 0, stream);
    });
}

sc_status sc_causal_conv_bwd_ntt_i32(const int32_t* dr, const int32_t* v, const int32_t* g,
                                     int32_t* dv, int32_t* dg, int64_t B, int64_t C, int64_t L,
                                     hipStream_t stream)
{
    return guarded([&] {
        return run_bwd(SC_KIND_NTT_I32, dr, v, g, dv, dg, B, C, L, nullptr, nullptr, 0, stream);
    });
}

sc_status sc_causal_conv_bwd_ex(sc_kind kind, const void* dr, const void* v, const void* g,
                                void* dv, void* dg, int64_t B, int64_t C, int64_t L,
                                const sc_options* opt, void* ws, size_t ws_bytes,
                                hipStream_t stream)
{
    return guarded(
        [&] { return run_bwd(kind, dr, v, g, dv, dg, B, C, L, opt, ws, ws_bytes, stream); });
}

sc_status sc_causal_conv_fixed_f32(const float* v, const float* g, float* r, int64_t B,
                                   int64_t C, int64_t L, int32_t frac_v, int32_t frac_g,
                                   hipStream_t stream)
{
    return guarded([&] {
        sc_options o{SC_PATH_AUTO, -1, frac_v, frac_g, {0, 0, 0, 0}};
        return run(SC_KIND_FIXED_F32, v, g, r, B, C, L, &o, nullptr, 0, stream);
    });
}

sc_status sc_causal_conv_fixed_f32_ws(const float* v, const float* g, float* r, int64_t B,
                                      int64_t C, int64_t L, int32_t frac_v, int32_t frac_g,
                                      void* ws, size_t ws_bytes, hipStream_t stream)
{
    return guarded([&] {
        sc_options o{SC_PATH_AUTO, -1, frac_v, frac_g, {0, 0, 0, 0}};
        return run(SC_KIND_FIXED_F32, v, g, r, B, C, L, &o, ws, ws_bytes, stream);
    });
}

int sc_fixed_range_ok(double max_abs_v, double max_abs_g, int32_t frac_v, int32_t frac_g,
                      int64_t L)
{
    if (!(max_abs_v >= 0) || !(max_abs_g >= 0) || L < 0) return 0;   // also rejects NaN
    if (frac_v < -kMaxFrac || frac_v > kMaxFrac || frac_g < -kMaxFrac || frac_g > kMaxFrac)
        return 0;
    // largest encodings: round(x 2^f) <= ceil(x 2^f); each must stay below 2^51
    const double bv = std::ceil(std::ldexp(max_abs_v, frac_v));
    const double bg = std::ceil(std::ldexp(max_abs_g, frac_g));
    if (!(bv < 0x1p51) || !(bg < 0x1p51)) return 0;
    // L * bv * bg <= (A B C - 1) / 2, in 128-bit integers (bv, bg < 2^51, L < 2^63)
    const unsigned __int128 P = (unsigned __int128)sc::NTT_PRIMES[0] * sc::NTT_PRIMES[1] *
                                sc::NTT_PRIMES[2];
    const unsigned __int128 prod = (unsigned __int128)(uint64_t)bv * (uint64_t)bg;
    if (prod != 0 && (unsigned __int128)L > ((P - 1) / 2) / prod) return 0;
    return 1;
}

// ---- filter shared by the batch

size_t sc_filter_spectrum_bytes(int64_t C, int64_t L)
{
    if (C < 0 || L < 1 || L > kMaxLFused) return 0;
    const int M = (int)std::max<int64_t>(64, next_pow2(L));
    const __int128 bytes = (__int128)C * sc::shared_spec_stride(M) * (int64_t)sizeof(float2);
    return bytes > (__int128)INT64_MAX ? 0 : (size_t)bytes;
}

namespace {

sc_status spectrum_run(sc_kind kind, const void* k, void* spec, int64_t C, int64_t L,
                       hipStream_t stream)
{
    if (kind != SC_KIND_F32 && kind != SC_KIND_BF16) return SC_ERR_INVALID_ARGUMENT;
    if (C < 0 || L < 0) return SC_ERR_INVALID_ARGUMENT;
    if (L > kMaxLFused) return SC_ERR_UNSUPPORTED;
    if (C == 0 || L == 0) return SC_OK;
    const size_t es = elt_size(kind);
    if ((__int128)C * L * (int64_t)es >= ((__int128)1 << 31)) return SC_ERR_UNSUPPORTED;
    if (!k || !spec) return SC_ERR_INVALID_ARGUMENT;
    if ((uintptr_t)k % es || (uintptr_t)spec % sizeof(float2)) return SC_ERR_INVALID_ARGUMENT;
    const size_t sbytes = sc_filter_spectrum_bytes(C, L);
    if ((uintptr_t)k < (uintptr_t)spec + sbytes && (uintptr_t)spec < (uintptr_t)k + C * L * es)
        return SC_ERR_INVALID_ARGUMENT;
    DeviceState* d = nullptr;
    sc_status st = device_state(&d, false, stream);
    if (st != SC_OK) return st;
    const int M = (int)std::max<int64_t>(64, next_pow2(L));
    const sc::Store s = kind == SC_KIND_F32 ? sc::Store::F32 : sc::Store::BF16;
    return sc::launch_shared_spectrum(s, k, (float2*)spec, (int)C, (int)L, M, d->fused_tw,
                                      stream) == hipSuccess
               ? SC_OK
               : SC_ERR_HIP;
}

// checks of an apply call; *n receives B*C*L
sc_status apply_check(sc_kind kind, const void* v, const void* spec, const void* r, int64_t B,
                      int64_t C, int64_t L, int64_t* n)
{
    if (kind != SC_KIND_F32 && kind != SC_KIND_BF16) return SC_ERR_INVALID_ARGUMENT;
    sc_status st = check_shape(kind, B, C, L, n);
    if (st != SC_OK) return st;
    if (L > kMaxLFused) return SC_ERR_UNSUPPORTED;
    if (*n == 0) return SC_OK;
    const size_t es = elt_size(kind);
    if ((__int128)C * L * (int64_t)es >= ((__int128)1 << 31)) return SC_ERR_UNSUPPORTED;
    if (!v || !spec || !r) return SC_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)v | (uintptr_t)r) % es || (uintptr_t)spec % sizeof(float2))
        return SC_ERR_INVALID_ARGUMENT;
    const uint64_t bytes = (uint64_t)*n * es;
    if (overlaps(r, v, bytes)) return SC_ERR_INVALID_ARGUMENT;
    const uint64_t sb = sc_filter_spectrum_bytes(C, L);
    if ((uintptr_t)r < (uintptr_t)spec + sb && (uintptr_t)spec < (uintptr_t)r + bytes)
        return SC_ERR_INVALID_ARGUMENT;
    return SC_OK;
}

// batch rows per launch so that one launch's v and r stay below 2^31 bytes
sc_status apply_run(sc_kind kind, const void* v, const void* spec, void* r, int64_t B, int64_t C,
                    int64_t L, hipStream_t stream, bool rev = false)
{
    DeviceState* d = nullptr;
    sc_status st = device_state(&d, false, stream);
    if (st != SC_OK) return st;
    const int M = (int)std::max<int64_t>(64, next_pow2(L));
    const sc::Store s = kind == SC_KIND_F32 ? sc::Store::F32 : sc::Store::BF16;
    const size_t es = elt_size(kind);
    const int64_t row = C * L * (int64_t)es;
    const int64_t rows = std::max<int64_t>(1, std::min<int64_t>(B, (((int64_t)1 << 31) - 1) / row));
    for (int64_t b0 = 0; b0 < B; b0 += rows) {
        const int64_t nb = std::min<int64_t>(rows, B - b0);
        const hipError_t e = sc::launch_shared_apply(
            s, (const char*)v + b0 * row, (const float2*)spec, (char*)r + b0 * row, (int)nb,
            (int)C, (int)L, M, kDefaultHead, rev, d->fused_tw, stream);
        if (e != hipSuccess) return SC_ERR_HIP;
    }
    return SC_OK;
}

sc_status shared_run(sc_kind kind, const void* v, const void* k, void* r, int64_t B, int64_t C,
                     int64_t L, hipStream_t stream)
{
    int64_t n = 0;
    // k plays the role of the spectrum in the checks; its own layout is checked below
    sc_status st = check_shape(kind, B, C, L, &n);
    if (st != SC_OK) return st;
    if (kind != SC_KIND_F32 && kind != SC_KIND_BF16) return SC_ERR_INVALID_ARGUMENT;
    if (L > kMaxLFused) return SC_ERR_UNSUPPORTED;
    if (n == 0) return SC_OK;
    const size_t es = elt_size(kind);
    if (!v || !k || !r) return SC_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)v | (uintptr_t)k | (uintptr_t)r) % es) return SC_ERR_INVALID_ARGUMENT;
    if ((__int128)C * L * (int64_t)es >= ((__int128)1 << 31)) return SC_ERR_UNSUPPORTED;
    if (overlaps(r, v, (uint64_t)n * es)) return SC_ERR_INVALID_ARGUMENT;
    if ((uintptr_t)r < (uintptr_t)k + C * L * es && (uintptr_t)k < (uintptr_t)r + n * es)
        return SC_ERR_INVALID_ARGUMENT;
    void* spec = nullptr;
    if (hipMallocAsync(&spec, sc_filter_spectrum_bytes(C, L), stream) != hipSuccess)
        return SC_ERR_HIP;
    st = spectrum_run(kind, k, spec, C, L, stream);
    if (st == SC_OK) st = apply_run(kind, v, spec, r, B, C, L, stream);
    if (hipFreeAsync(spec, stream) != hipSuccess && st == SC_OK) st = SC_ERR_HIP;
    return st;
}

// gradients for a filter shared by the batch: dv from the spectrum (made here from k when
// spec is null), dk by the batch-summing kernel
sc_status shared_bwd_run(sc_kind kind, const void* dr, const void* v, const void* k,
                         const void* spec, void* dv, void* dk, int64_t B, int64_t C, int64_t L,
                         hipStream_t stream)
{
    int64_t n = 0;
    sc_status st = check_shape(kind, B, C, L, &n);
    if (st != SC_OK) return st;
    if (kind != SC_KIND_F32 && kind != SC_KIND_BF16) return SC_ERR_INVALID_ARGUMENT;
    if (L > kMaxLFused) return SC_ERR_UNSUPPORTED;
    const size_t es = elt_size(kind);
    if ((__int128)C * L * (int64_t)es >= ((__int128)1 << 31)) return SC_ERR_UNSUPPORTED;
    if (n == 0) {
        // no rows: dv is empty, and dk (C x L, when that is not empty) is the sum over no
        // rows, zero
        if (C == 0 || L == 0) return SC_OK;
        if (!dk || (uintptr_t)dk % es) return SC_ERR_INVALID_ARGUMENT;
        return sc::launch_zero16(dk, C * L * (int64_t)(es / 2), stream) == hipSuccess
                   ? SC_OK
                   : SC_ERR_HIP;
    }
    // the row loops count batch rows in 32 bits
    if (B > INT32_MAX) return SC_ERR_UNSUPPORTED;
    const void* filt = spec ? spec : k;
    if (!dr || !v || !filt || !dv || !dk) return SC_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)dr | (uintptr_t)v | (uintptr_t)dv | (uintptr_t)dk) % es)
        return SC_ERR_INVALID_ARGUMENT;
    if (spec ? (uintptr_t)spec % sizeof(float2) : (uintptr_t)k % es) return SC_ERR_INVALID_ARGUMENT;
    const uint64_t nb = (uint64_t)n * es, kb = (uint64_t)(C * L) * es;
    const uint64_t fb = spec ? sc_filter_spectrum_bytes(C, L) : kb;
    struct Buf { const void* p; uint64_t b; };
    const Buf ins[3] = {{dr, nb}, {v, nb}, {filt, fb}};
    const Buf outs[2] = {{dv, nb}, {dk, kb}};
    for (const Buf& o : outs)
        for (const Buf& i : ins)
            if ((uintptr_t)o.p < (uintptr_t)i.p + i.b && (uintptr_t)i.p < (uintptr_t)o.p + o.b)
                return SC_ERR_INVALID_ARGUMENT;
    if ((uintptr_t)dv < (uintptr_t)dk + kb && (uintptr_t)dk < (uintptr_t)dv + nb)
        return SC_ERR_INVALID_ARGUMENT;
    DeviceState* d = nullptr;
    st = device_state(&d, false, stream);
    if (st != SC_OK) return st;
    void* own = nullptr;
    if (!spec) {
        if (hipMallocAsync(&own, sc_filter_spectrum_bytes(C, L), stream) != hipSuccess)
            return SC_ERR_HIP;
        st = spectrum_run(kind, k, own, C, L, stream);
        spec = own;
    }
    if (st == SC_OK) {
        const int M = (int)std::max<int64_t>(64, next_pow2(L));
        const sc::Store s = kind == SC_KIND_F32 ? sc::Store::F32 : sc::Store::BF16;
        if (sc::shared_bwd_blocks(C, M) >= kSharedBwdMinBlocks) {
            // one kernel: dv and dk from the same transform per row
            const bool pair = L % 2 == 0 && ((uintptr_t)dk | (uintptr_t)dv) % (2 * es) == 0;
            if (sc::launch_shared_bwd(s, dr, v, (const float2*)spec, dv, dk, (int)B, (int)C,
                                      (int)L, M, kDefaultHead, pair, d->fused_tw,
                                      stream) != hipSuccess)
                st = SC_ERR_HIP;
        } else {
            // too few channel groups to fill the GPU with the row loop alone: dv by the
            // apply kernel on every row pair, dk by the row-looping kernel
            st = apply_run(kind, dr, spec, dv, B, C, L, stream, true);
            const bool pair = L % 2 == 0 && (uintptr_t)dk % (2 * es) == 0;
            if (st == SC_OK &&
                sc::launch_shared_dk(s, dr, v, dk, (int)B, (int)C, (int)L, M, kDefaultHead, pair,
                                     d->fused_tw, stream) != hipSuccess)
                st = SC_ERR_HIP;
        }
    }
    if (own && hipFreeAsync(own, stream) != hipSuccess && st == SC_OK) st = SC_ERR_HIP;
    return st;
}

}  // namespace

sc_status sc_causal_conv_spec_bwd_f32(const float* dr, const float* v, const void* spec,
                                      float* dv, float* dk, int64_t B, int64_t C, int64_t L,
                                      hipStream_t stream)
{
    return guarded([&] {
        return shared_bwd_run(SC_KIND_F32, dr, v, nullptr, spec, dv, dk, B, C, L, stream);
    });
}

sc_status sc_causal_conv_spec_bwd_bf16(const uint16_t* dr, const uint16_t* v, const void* spec,
                                       uint16_t* dv, uint16_t* dk, int64_t B, int64_t C,
                                       int64_t L, hipStream_t stream)
{
    return guarded([&] {
        return shared_bwd_run(SC_KIND_BF16, dr, v, nullptr, spec, dv, dk, B, C, L, stream);
    });
}

sc_status sc_causal_conv_shared_bwd_f32(const float* dr, const float* v, const float* k, float* dv,
                                        float* dk, int64_t B, int64_t C, int64_t L,
                                        hipStream_t stream)
{
    return guarded([&] {
        return shared_bwd_run(SC_KIND_F32, dr, v, k, nullptr, dv, dk, B, C, L, stream);
    });
}

sc_status sc_causal_conv_shared_bwd_bf16(const uint16_t* dr, const uint16_t* v, const uint16_t* k,
                                         uint16_t* dv, uint16_t* dk, int64_t B, int64_t C,
                                         int64_t L, hipStream_t stream)
{
    return guarded([&] {
        return shared_bwd_run(SC_KIND_BF16, dr, v, k, nullptr, dv, dk, B, C, L, stream);
    });
}

sc_status sc_filter_spectrum_f32(const float* k, void* spec, int64_t C, int64_t L,
                                 hipStream_t stream)
{
    return guarded([&] { return spectrum_run(SC_KIND_F32, k, spec, C, L, stream); });
}

sc_status sc_filter_spectrum_bf16(const uint16_t* k, void* spec, int64_t C, int64_t L,
                                  hipStream_t stream)
{
    return guarded([&] { return spectrum_run(SC_KIND_BF16, k, spec, C, L, stream); });
}

sc_status sc_causal_conv_spec_f32(const float* v, const void* spec, float* r, int64_t B,
                                  int64_t C, int64_t L, hipStream_t stream)
{
    return guarded([&] {
        int64_t n = 0;
        sc_status st = apply_check(SC_KIND_F32, v, spec, r, B, C, L, &n);
        if (st != SC_OK || n == 0) return st;
        return apply_run(SC_KIND_F32, v, spec, r, B, C, L, stream);
    });
}

sc_status sc_causal_conv_spec_bf16(const uint16_t* v, const void* spec, uint16_t* r, int64_t B,
                                   int64_t C, int64_t L, hipStream_t stream)
{
    return guarded([&] {
        int64_t n = 0;
        sc_status st = apply_check(SC_KIND_BF16, v, spec, r, B, C, L, &n);
        if (st != SC_OK || n == 0) return st;
        return apply_run(SC_KIND_BF16, v, spec, r, B, C, L, stream);
    });
}

sc_status sc_causal_conv_shared_f32(const float* v, const float* k, float* r, int64_t B,
                                    int64_t C, int64_t L, hipStream_t stream)
{
    return guarded([&] { return shared_run(SC_KIND_F32, v, k, r, B, C, L, stream); });
}

sc_status sc_causal_conv_shared_bf16(const uint16_t* v, const uint16_t* k, uint16_t* r, int64_t B,
                                     int64_t C, int64_t L, hipStream_t stream)
{
    return guarded([&] { return shared_run(SC_KIND_BF16, v, k, r, B, C, L, stream); });
}

int sc_ntt_range_ok(int64_t max_abs_v, int64_t max_abs_g, int64_t L)
{
    if (max_abs_v < 0 || max_abs_g < 0 || L < 0) return 0;
    const __int128 worst = (__int128)L * (__int128)max_abs_v * (__int128)max_abs_g;
    return worst <= (__int128)((kNttP - 1) / 2) ? 1 : 0;
}

const char* sc_status_string(sc_status s)
{
    switch (s) {
    case SC_OK: return "SC_OK";
    case SC_ERR_INVALID_ARGUMENT: return "SC_ERR_INVALID_ARGUMENT";
    case SC_ERR_UNSUPPORTED: return "SC_ERR_UNSUPPORTED";
    case SC_ERR_HIP: return "SC_ERR_HIP";
    case SC_ERR_WORKSPACE: return "SC_ERR_WORKSPACE";
    default: return "SC_STATUS_UNKNOWN";
    }
}

sc_status sc_causal_conv_noalloc(sc_kind kind, const void* v, const void* g, void* r,
                                 int64_t B, int64_t C, int64_t L, hipStream_t stream)
{
    return guarded([&] {
        if (kind != SC_KIND_F32 && kind != SC_KIND_BF16 && kind != SC_KIND_NTT_I32)
            return SC_ERR_INVALID_ARGUMENT;
        int64_t n = 0;
        sc_status st = check_args(kind, v, g, r, B, C, L, &n);
        if (st != SC_OK) return st;
        sc_path path;
        if ((st = resolve_path(kind, L, SC_PATH_AUTO, &path)) != SC_OK) return st;
        if (n == 0) return SC_OK;
        void* ws = nullptr;
        size_t ws_bytes = 0;
        if (path == SC_PATH_FOUR_STEP &&
            sc::static_scratch(&ws, &ws_bytes) != hipSuccess)
            return SC_ERR_HIP;
        const Job job{v, g, r};
        return run_jobs(kind, &job, 1, false, n, B, C, L, nullptr, ws, ws_bytes, stream, true);
    });
}

sc_status sc_prepare(sc_kind kind, int64_t L)
{
    return guarded([&] {
        int64_t n = 0;
        sc_status st = check_shape(kind, 1, 1, L, &n);
        if (st != SC_OK) return st;
        if (L == 0) return SC_OK;   // such a call enqueues nothing and needs no table
        sc_path path;
        if ((st = resolve_path(kind, L, SC_PATH_AUTO, &path)) != SC_OK) return st;
        DeviceState* d = nullptr;
        st = device_state(&d, exact_kind(kind), nullptr);
        if (st != SC_OK || path != SC_PATH_FOUR_STEP) return st;
        std::lock_guard<std::mutex> lk(g_mu);
        if (exact_kind(kind)) {
            const double* wtab = nullptr;
            for (int i = 0; i < (kind == SC_KIND_FIXED_F32 ? 3 : 1) && st == SC_OK; ++i)
                st = ntt4_table(*d, (int)next_pow2(L), i, &wtab, nullptr);
            return st;
        }
        sc::FsTw tw;
        return fourstep_tables(*d, (int)next_pow2(L), &tw, nullptr);
    });
}

int sc_version(void) { return 902; }

}  // extern "C"
