// kdn_abi.cpp -- the C ABI declared in include/kdn.h: host-side validation of
// every argument (before any HIP call), then one kernel launch on the
// caller's stream.
#include "kdn.h"
#include "kdn_launch.h"
#include "kdn_workspace.h"

#include <atomic>
#include <initializer_list>
#include <stdint.h>

namespace {

// Compute units of the current device, queried once per device (the value
// never changes; concurrent first calls store the same number).
int device_cus() {
    constexpr int MAXDEV = 64;
    static std::atomic<int> cache[MAXDEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAXDEV)
        return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges, empty ranges never overlap)
bool overlap(const void *a, long long na, const void *b, long long nb) {
    if (!a || !b || na <= 0 || nb <= 0)
        return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

bool valid_variant(int v) { return v >= KDN_DELTANET && v <= KDN_ISO_KDN; }
bool is_kdn(int v) { return v == KDN_DIAG_KDN || v == KDN_ISO_KDN; }
// float32 variances per (sequence, head): d_k (diagonal KDN), 1 (isotropic)
long long p_per_head(int v, int d_k) {
    return v == KDN_DIAG_KDN ? d_k : (v == KDN_ISO_KDN ? 1 : 0);
}
// Alignment of the variance tensors: vectors of d_k floats 16 bytes, the
// per-head scalar of isotropic KDN one float.
uintptr_t p_align(int v) { return v == KDN_ISO_KDN ? 4 : 16; }
bool valid_dtype(int d) { return d == KDN_F32 || d == KDN_BF16; }
bool valid_dim(int d) { return d == 64 || d == 128; }

// Gate pointers the variant does not use must be NULL; the ones it uses must
// be non-NULL unless the per-token tensors are empty.
kdn_status check_gates(int variant, const void *alpha, const void *beta,
                       const void *xi, const void *r, bool empty) {
    const bool need_alpha = variant != KDN_DELTANET;
    const bool kdn = is_kdn(variant);
    if (!need_alpha && alpha) return KDN_ERR_NULL;
    if (kdn && beta) return KDN_ERR_NULL;
    if (!kdn && (xi || r)) return KDN_ERR_NULL;
    if (empty) return KDN_OK;
    if (need_alpha && !alpha) return KDN_ERR_NULL;
    if (!kdn && !beta) return KDN_ERR_NULL;
    if (kdn && (!xi || !r)) return KDN_ERR_NULL;
    return KDN_OK;
}

}  // namespace

extern "C" {

int kdn_abi_version(void) { return KDN_ABI_VERSION; }

const char *kdn_status_string(kdn_status s) {
    switch (s) {
    case KDN_OK: return "ok";
    case KDN_ERR_NULL: return "a required pointer is NULL, or a pointer the variant does not use is set";
    case KDN_ERR_SHAPE: return "negative or overflowing sizes";
    case KDN_ERR_UNSUPPORTED: return "unsupported variant, dtype, head dimension or chunk length";
    case KDN_ERR_ALIGN: return "a pointer is not aligned as required";
    case KDN_ERR_ALIAS: return "an output overlaps an input it may not overlap";
    case KDN_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case KDN_ERR_WORKSPACE: return "the workspace is smaller than kdn_chunk_prefill_workspace_size";
    case KDN_ERR_SCRATCH: return "one chunk of every head of a sequence needs more than the library's static scratch";
    }
    return "unknown status";
}

int kdn_chunk_prefill_chunk_size(kdn_dtype dtype, int d_k, int d_v, int chunk) {
    if (!valid_dtype(dtype) || !valid_dim(d_k) || !valid_dim(d_v))
        return -1;
    if (chunk == 0)
        chunk = (dtype == KDN_F32 && d_k == 128) ? 32 : 64;
    if (chunk != 32 && chunk != 64)
        return -1;
    if (dtype == KDN_F32 && d_k == 128 && chunk == 64)
        return -1;   // float32 operands of a 64 x 128 chunk exceed the LDS
    return chunk;
}

// Shape checks shared by kdn_chunk_prefill and its workspace query; the
// chunk length in use goes to *C.
static kdn_status prefill_shape(int variant, int dtype, int B, int T, int H, int d_k,
                                int d_v, int chunk, int *C) {
    if (!valid_variant(variant) || !valid_dtype(dtype))
        return KDN_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H < 0 || d_k <= 0 || d_v <= 0)
        return KDN_ERR_SHAPE;
    const long long bh = (long long)B * H;
    const long long tok = bh * T;
    if (bh * d_k * d_v >= (1LL << 31) || tok * (d_k > d_v ? d_k : d_v) >= (1LL << 40))
        return KDN_ERR_SHAPE;
    if (!valid_dim(d_k) || !valid_dim(d_v))
        return KDN_ERR_UNSUPPORTED;
    *C = kdn_chunk_prefill_chunk_size((kdn_dtype)dtype, d_k, d_v, chunk);
    if (*C < 0)
        return KDN_ERR_UNSUPPORTED;
    return KDN_OK;
}

unsigned long long kdn_chunk_prefill_workspace_size(kdn_variant variant, kdn_dtype dtype,
                                                    int B, int T, int H, int d_k,
                                                    int d_v, int chunk,
                                                    kdn_status *status) {
    int C = 0;
    const kdn_status st = prefill_shape(variant, dtype, B, T, H, d_k, d_v, chunk, &C);
    if (status)
        *status = st;
    if (st != KDN_OK || (long long)B * H * T == 0)
        return 0;
    return (unsigned long long)kdn::prefill_workspace_bytes(variant, dtype == KDN_BF16, B, T,
                                                            H, d_k, C);
}

}  // extern "C"

// Every argument check of kdn_chunk_prefill except the workspace's own (size,
// alignment, overlap); `workspace` says whether the call has one (the
// in-place variance rule depends on it).  No HIP call.
kdn_status kdn::prefill_check(int variant, int dtype, int B, int T, int H, int d_k, int d_v,
                              int chunk, const void *q, const void *k, const void *v,
                              const void *alpha, const void *beta, const void *proc_noise,
                              const void *obs_noise, const float *S0, const float *p0,
                              const void *o, const float *S_out, const float *p_out,
                              bool workspace, int *C_out) {
    int C = 0;
    if (kdn_status st = prefill_shape(variant, dtype, B, T, H, d_k, d_v, chunk, &C))
        return st;
    const long long bh = (long long)B * H;
    const long long tok = bh * T;
    const bool kdn = is_kdn(variant);
    // Empty tensors may be passed as NULL (a zero-size torch tensor has no
    // storage): per-token tensors when B*H*T = 0, state tensors when B*H = 0.
    if (tok > 0 && (!q || !k || !v || !o))
        return KDN_ERR_NULL;
    if (kdn_status st = check_gates(variant, alpha, beta, proc_noise, obs_noise, tok == 0))
        return st;
    if (bh > 0 && !S_out)
        return KDN_ERR_NULL;
    if (kdn && bh > 0 && (!p0 || !p_out))
        return KDN_ERR_NULL;
    if (!kdn && (p0 || p_out))
        return KDN_ERR_NULL;
    const long long es = dtype == KDN_BF16 ? 2 : 4;
    // vectors of d_k / d_v elements: 16 bytes; per-head scalars: one element
    const void *vec[] = {q, k, v, variant == KDN_GATED_DELTANET ? nullptr : alpha,
                         proc_noise, S0, o, S_out};
    const void *sca[] = {beta, obs_noise, variant == KDN_GATED_DELTANET ? alpha : nullptr};
    for (const void *x : vec)
        if (x && !aligned(x, 16))
            return KDN_ERR_ALIGN;
    for (const void *x : sca)
        if (x && !aligned(x, (uintptr_t)es))
            return KDN_ERR_ALIGN;
    for (const void *x : {(const void *)p0, (const void *)p_out})
        if (x && !aligned(x, p_align(variant)))
            return KDN_ERR_ALIGN;

    const long long n_qk = tok * d_k * es, n_v = tok * d_v * es;
    const long long n_a = variant == KDN_GATED_DELTANET ? tok * es
                        : (variant == KDN_DELTANET ? 0 : tok * d_k * es);
    const long long n_b = kdn ? 0 : tok * es;
    const long long n_x = kdn ? tok * d_k * es : 0, n_r = kdn ? tok * es : 0;
    const long long n_S = bh * d_k * d_v * 4, n_p = bh * p_per_head(variant, d_k) * 4;
    // o overlaps no input; S_out may be S0 exactly (every workgroup reads its
    // slice of S0 before it writes the same slice).  p_out may be p0 exactly
    // with a workspace (the variance scan reads each entry of p0 in the thread
    // that later writes it) or without tokens; the single-pass kernel reads p0
    // in every value-block workgroup of a head and writes p_out from one of
    // them, so there it must lie elsewhere.
    const bool p_in_place = kdn && p0 && p_out == p0 && (tok == 0 || workspace);
    struct R { const void *p; long long n; } ins[] = {
        {q, n_qk}, {k, n_qk}, {v, n_v}, {alpha, n_a}, {beta, n_b},
        {proc_noise, n_x}, {obs_noise, n_r}, {S0, n_S}, {p0, n_p}};
    for (const R &x : ins) {
        if (overlap(o, tok * d_v * es, x.p, x.n)) return KDN_ERR_ALIAS;
        if (x.p != S0 && overlap(S_out, n_S, x.p, x.n)) return KDN_ERR_ALIAS;
        if (kdn && !(p_in_place && x.p == p0) && overlap(p_out, n_p, x.p, x.n))
            return KDN_ERR_ALIAS;
    }
    if (S0 && S0 != S_out && overlap(S_out, n_S, S0, n_S)) return KDN_ERR_ALIAS;
    if (overlap(o, tok * d_v * es, S_out, n_S)) return KDN_ERR_ALIAS;
    if (kdn && (overlap(o, tok * d_v * es, p_out, n_p) || overlap(S_out, n_S, p_out, n_p)))
        return KDN_ERR_ALIAS;
    *C_out = C;
    return KDN_OK;
}

extern "C" {

kdn_status kdn_chunk_prefill(kdn_variant variant, kdn_dtype dtype, int B, int T,
                             int H, int d_k, int d_v, int chunk, float mu,
                             const void *q, const void *k, const void *v,
                             const void *alpha, const void *beta,
                             const void *proc_noise, const void *obs_noise,
                             const float *S0, const float *p0, void *o,
                             float *S_out, float *p_out, void *workspace,
                             unsigned long long workspace_bytes, void *stream) {
    int C = 0;
    if (kdn_status st = kdn::prefill_check(variant, dtype, B, T, H, d_k, d_v, chunk, q, k, v,
                                           alpha, beta, proc_noise, obs_noise, S0, p0, o,
                                           S_out, p_out, workspace != nullptr, &C))
        return st;
    const long long bh = (long long)B * H;
    const long long tok = bh * T;
    const bool kdn = is_kdn(variant);
    const long long es = dtype == KDN_BF16 ? 2 : 4;
    const long long n_qk = tok * d_k * es, n_v = tok * d_v * es;
    const long long n_a = variant == KDN_GATED_DELTANET ? tok * es
                        : (variant == KDN_DELTANET ? 0 : tok * d_k * es);
    const long long n_b = kdn ? 0 : tok * es;
    const long long n_x = kdn ? tok * d_k * es : 0, n_r = kdn ? tok * es : 0;
    const long long n_S = bh * d_k * d_v * 4, n_p = bh * p_per_head(variant, d_k) * 4;
    struct R { const void *p; long long n; } ins[] = {
        {q, n_qk}, {k, n_qk}, {v, n_v}, {alpha, n_a}, {beta, n_b},
        {proc_noise, n_x}, {obs_noise, n_r}, {S0, n_S}, {p0, n_p}};
    // Workspace of the two-pass schedule: none when there is nothing to do.
    long long n_ws = 0;
    if (workspace && tok > 0) {
        n_ws = kdn::prefill_workspace_bytes(variant, dtype == KDN_BF16, B, T, H, d_k, C);
        if ((long long)workspace_bytes < n_ws)
            return KDN_ERR_WORKSPACE;
        if (!aligned(workspace, 256))
            return KDN_ERR_ALIGN;
        const R outs[] = {{o, tok * d_v * es}, {S_out, n_S}, {p_out, n_p}};
        for (const R &x : ins)
            if (overlap(workspace, n_ws, x.p, x.n)) return KDN_ERR_ALIAS;
        for (const R &x : outs)
            if (overlap(workspace, n_ws, x.p, x.n)) return KDN_ERR_ALIAS;
    }

    kdn::PrefillParams P;
    P.variant = variant;
    P.bf16 = dtype == KDN_BF16;
    P.B = B; P.T = T; P.H = H; P.dk = d_k; P.dv = d_v; P.chunk = C;
    P.mu = mu;
    P.q = q; P.k = k; P.v = v; P.alpha = alpha; P.beta = beta;
    P.xi = proc_noise; P.r = obs_noise;
    P.S0 = S0; P.p0 = p0; P.o = o; P.S_out = S_out; P.p_out = p_out;
    P.ws = nullptr; P.ws_mob = nullptr; P.ws_p0 = nullptr; P.ws_pre = nullptr;
    P.ws_stat = nullptr;
    // bf16 two-pass: permuted records for the chain kernel
    P.rec_perm = (n_ws > 0 && dtype == KDN_BF16) ? 1 : 0;
    P.states = nullptr;
    P.beta_out = nullptr;
    P.w_out = nullptr;
    P.invs_out = nullptr;
    P.cus = device_cus();
    if (n_ws > 0) {
        P.ws = workspace;
        const long long nc = kdn::num_chunks(T, C);
        char *base = static_cast<char *>(workspace) +
                     kdn::WsLayout::make(dtype == KDN_BF16, C, d_k).records(bh, nc);
        if (variant == KDN_DIAG_KDN) {
            const long long n_mob = kdn::WsLayout::mobius_bytes(bh, nc, d_k);
            P.ws_mob = reinterpret_cast<float *>(base);
            P.ws_p0 = reinterpret_cast<float *>(base + n_mob);
            P.ws_pre = reinterpret_cast<float *>(base + n_mob +
                                                 kdn::WsLayout::p0_bytes(bh, nc, d_k));
        } else if (variant == KDN_ISO_KDN) {
            const long long n_mob = kdn::WsLayout::mobius_bytes(bh, nc, 1);
            P.ws_mob = reinterpret_cast<float *>(base);
            P.ws_stat = reinterpret_cast<float *>(base + n_mob);
            P.ws_p0 = reinterpret_cast<float *>(base + n_mob +
                                                kdn::WsLayout::stat_bytes(bh, nc, C));
        }
    }
    const hipError_t e = kdn::launch_prefill(P, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDN_OK : KDN_ERR_HIP;
}

kdn_status kdn_recurrent_decode(kdn_variant variant, kdn_dtype dtype, int N, int H,
                                int d_k, int d_v, float mu, const void *q,
                                const void *k, const void *v, const void *alpha,
                                const void *beta, const void *proc_noise,
                                const void *obs_noise, float *S, float *p, void *o,
                                void *stream) {
    if (!valid_variant(variant) || !valid_dtype(dtype))
        return KDN_ERR_UNSUPPORTED;
    if (N < 0 || H < 0 || d_k <= 0 || d_v <= 0)
        return KDN_ERR_SHAPE;
    const long long nh = (long long)N * H;
    if (nh * d_k * d_v >= (1LL << 31))
        return KDN_ERR_SHAPE;
    if (!valid_dim(d_k) || !valid_dim(d_v))
        return KDN_ERR_UNSUPPORTED;
    const bool kdn = is_kdn(variant);
    if (nh > 0 && (!q || !k || !v || !o || !S))
        return KDN_ERR_NULL;
    if (kdn_status st = check_gates(variant, alpha, beta, proc_noise, obs_noise, nh == 0))
        return st;
    if (!kdn && p)
        return KDN_ERR_NULL;
    if (kdn && nh > 0 && !p)
        return KDN_ERR_NULL;
    const long long es = dtype == KDN_BF16 ? 2 : 4;
    const void *vec[] = {q, k, v, variant == KDN_GATED_DELTANET ? nullptr : alpha,
                         proc_noise, S, o};
    const void *sca[] = {beta, obs_noise, variant == KDN_GATED_DELTANET ? alpha : nullptr};
    for (const void *x : vec)
        if (x && !aligned(x, 16))
            return KDN_ERR_ALIGN;
    for (const void *x : sca)
        if (x && !aligned(x, (uintptr_t)es))
            return KDN_ERR_ALIGN;
    if (p && !aligned(p, p_align(variant)))
        return KDN_ERR_ALIGN;

    const long long n_qk = nh * d_k * es, n_v = nh * d_v * es;
    const long long n_a = variant == KDN_GATED_DELTANET ? nh * es
                        : (variant == KDN_DELTANET ? 0 : nh * d_k * es);
    const long long n_b = kdn ? 0 : nh * es;
    const long long n_x = kdn ? nh * d_k * es : 0, n_r = kdn ? nh * es : 0;
    const long long n_S = nh * d_k * d_v * 4, n_p = nh * p_per_head(variant, d_k) * 4;
    const long long n_o = nh * d_v * es;
    struct R { const void *p; long long n; } ins[] = {
        {q, n_qk}, {k, n_qk}, {v, n_v}, {alpha, n_a}, {beta, n_b},
        {proc_noise, n_x}, {obs_noise, n_r}};
    for (const R &x : ins) {
        if (overlap(o, n_o, x.p, x.n)) return KDN_ERR_ALIAS;
        if (overlap(S, n_S, x.p, x.n)) return KDN_ERR_ALIAS;
        if (kdn && overlap(p, n_p, x.p, x.n)) return KDN_ERR_ALIAS;
    }
    if (overlap(o, n_o, S, n_S) || (kdn && (overlap(o, n_o, p, n_p) ||
                                            overlap(S, n_S, p, n_p))))
        return KDN_ERR_ALIAS;

    kdn::DecodeParams P;
    P.variant = variant;
    P.bf16 = dtype == KDN_BF16;
    P.N = N; P.H = H; P.dk = d_k; P.dv = d_v; P.mu = mu;
    P.q = q; P.k = k; P.v = v; P.alpha = alpha; P.beta = beta;
    P.xi = proc_noise; P.r = obs_noise;
    P.T = 1;
    P.S0 = S; P.p0 = p; P.S = S; P.p = p; P.o = o;
    const hipError_t e = kdn::launch_decode(P, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDN_OK : KDN_ERR_HIP;
}

kdn_status kdn_recurrent_decode_multi(kdn_variant variant, kdn_dtype dtype, int N, int T,
                                      int H, int d_k, int d_v, float mu, const void *q,
                                      const void *k, const void *v, const void *alpha,
                                      const void *beta, const void *proc_noise,
                                      const void *obs_noise, const float *S0,
                                      const float *p0, void *o, float *S_out,
                                      float *p_out, void *stream) {
    if (!valid_variant(variant) || !valid_dtype(dtype))
        return KDN_ERR_UNSUPPORTED;
    if (N < 0 || T < 0 || H < 0 || d_k <= 0 || d_v <= 0)
        return KDN_ERR_SHAPE;
    const long long nh = (long long)N * H;
    const long long tok = nh * T;
    if (nh * d_k * d_v >= (1LL << 31) || tok * (d_k > d_v ? d_k : d_v) >= (1LL << 40))
        return KDN_ERR_SHAPE;
    if (!valid_dim(d_k) || !valid_dim(d_v))
        return KDN_ERR_UNSUPPORTED;
    const bool kdn = is_kdn(variant);
    if (tok > 0 && (!q || !k || !v || !o))
        return KDN_ERR_NULL;
    if (kdn_status st = check_gates(variant, alpha, beta, proc_noise, obs_noise, tok == 0))
        return st;
    if (nh > 0 && !S_out)
        return KDN_ERR_NULL;
    if (kdn && nh > 0 && (!p0 || !p_out))
        return KDN_ERR_NULL;
    if (!kdn && (p0 || p_out))
        return KDN_ERR_NULL;
    const long long es = dtype == KDN_BF16 ? 2 : 4;
    const void *vec[] = {q, k, v, variant == KDN_GATED_DELTANET ? nullptr : alpha,
                         proc_noise, S0, o, S_out};
    const void *sca[] = {beta, obs_noise, variant == KDN_GATED_DELTANET ? alpha : nullptr};
    for (const void *x : vec)
        if (x && !aligned(x, 16))
            return KDN_ERR_ALIGN;
    for (const void *x : sca)
        if (x && !aligned(x, (uintptr_t)es))
            return KDN_ERR_ALIGN;
    for (const void *x : {(const void *)p0, (const void *)p_out})
        if (x && !aligned(x, p_align(variant)))
            return KDN_ERR_ALIGN;

    const long long n_qk = tok * d_k * es, n_v = tok * d_v * es;
    const long long n_a = variant == KDN_GATED_DELTANET ? tok * es
                        : (variant == KDN_DELTANET ? 0 : tok * d_k * es);
    const long long n_b = kdn ? 0 : tok * es;
    const long long n_x = kdn ? tok * d_k * es : 0, n_r = kdn ? tok * es : 0;
    const long long n_S = nh * d_k * d_v * 4, n_p = nh * p_per_head(variant, d_k) * 4;
    const long long n_o = tok * d_v * es;
    // o overlaps nothing; S_out may be S0 exactly and p_out may be p0 exactly
    // (each workgroup reads its slice before writing it); no other overlap.
    struct R { const void *p; long long n; } ins[] = {
        {q, n_qk}, {k, n_qk}, {v, n_v}, {alpha, n_a}, {beta, n_b},
        {proc_noise, n_x}, {obs_noise, n_r}, {S0, n_S}, {p0, n_p}};
    for (const R &x : ins) {
        if (overlap(o, n_o, x.p, x.n)) return KDN_ERR_ALIAS;
        if (x.p != S0 && overlap(S_out, n_S, x.p, x.n)) return KDN_ERR_ALIAS;
        if (kdn && x.p != p0 && overlap(p_out, n_p, x.p, x.n)) return KDN_ERR_ALIAS;
    }
    if (S0 && S0 != S_out && overlap(S_out, n_S, S0, n_S)) return KDN_ERR_ALIAS;
    if (kdn && p0 != p_out && overlap(p_out, n_p, p0, n_p)) return KDN_ERR_ALIAS;
    if (overlap(o, n_o, S_out, n_S)) return KDN_ERR_ALIAS;
    if (kdn && (overlap(o, n_o, p_out, n_p) || overlap(S_out, n_S, p_out, n_p)))
        return KDN_ERR_ALIAS;

    kdn::DecodeParams P;
    P.variant = variant;
    P.bf16 = dtype == KDN_BF16;
    P.N = N; P.H = H; P.dk = d_k; P.dv = d_v; P.T = T; P.mu = mu;
    P.q = q; P.k = k; P.v = v; P.alpha = alpha; P.beta = beta;
    P.xi = proc_noise; P.r = obs_noise;
    P.S0 = S0; P.p0 = p0; P.S = S_out; P.p = p_out; P.o = o;
    const hipError_t e = kdn::launch_decode_multi(P, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDN_OK : KDN_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Gradients of the chunkwise prefill.
// ---------------------------------------------------------------------------
namespace {
// Workspace of the gradient call, sections 256-byte aligned: the forward's
// two-pass workspace, S at every chunk start, dS at every chunk end; for
// isotropic KDN the derived write strengths and their gradients, for
// diagonal KDN the gains and their gradients, 1/s and sum_i w_i dw_i per
// token and the variance before every token; for both the variance chain's
// chunk maps and its gradient at every chunk end.
struct BwdWs {
    long long fwd, states, dstates, beta, dbeta, w, dw, invs, wdw, pp, cmap, cdp, total;
};
long long up256(long long n) { return (n + 255) / 256 * 256; }
BwdWs backward_ws(int variant, int bf16, long long B, long long T, long long H, int d_k,
                  int d_v, int C) {
    BwdWs w{};
    const long long bh = B * H, nc = kdn::num_chunks(T, C), tok = bh * T;
    if (tok == 0)
        return w;
    const bool iso = variant == KDN_ISO_KDN, diag = variant == KDN_DIAG_KDN;
    long long o = up256(kdn::prefill_workspace_bytes(variant, bf16, B, T, H, d_k, C));
    w.fwd = 0;
    const long long es = bf16 ? 2 : 4;                 // saved states: the call dtype
    w.states = o;  o += up256(bh * nc * d_k * d_v * es);
    w.dstates = o; o += up256(bh * nc * d_k * d_v * es);
    if (iso) {
        w.beta = o;  o += up256(tok * 4);
        w.dbeta = o; o += up256(tok * 4);
        w.cmap = o;  o += up256(bh * nc * 8);
        w.cdp = o;   o += up256(bh * nc * 4);
    }
    if (diag) {
        w.w = o;     o += up256(tok * d_k * 4);
        w.dw = o;    o += up256(tok * d_k * 4);
        w.invs = o;  o += up256(tok * 4);
        w.wdw = o;   o += up256(tok * 4);
        w.pp = o;    o += up256(tok * d_k * 4);
        w.cmap = o;  o += up256(bh * nc * d_k * 8);
        w.cdp = o;   o += up256(bh * nc * d_k * 4);
    }
    w.total = o;
    return w;
}
}  // namespace

unsigned long long kdn_chunk_prefill_backward_workspace_size(kdn_variant variant, kdn_dtype dtype,
                                                             int B, int T, int H, int d_k,
                                                             int d_v, int chunk,
                                                             kdn_status *status) {
    int C = 0;
    kdn_status st = prefill_shape(variant, dtype, B, T, H, d_k, d_v, chunk, &C);
    if (status)
        *status = st;
    if (st != KDN_OK)
        return 0;
    return (unsigned long long)backward_ws(variant, dtype == KDN_BF16, B, T, H, d_k, d_v, C).total;
}

kdn_status kdn_chunk_prefill_backward(kdn_variant variant, kdn_dtype dtype, int B, int T,
                                      int H, int d_k, int d_v, int chunk, float mu,
                                      const void *q, const void *k, const void *v,
                                      const void *alpha, const void *beta,
                                      const void *proc_noise, const void *obs_noise,
                                      const float *S0, const float *p0,
                                      const void *d_o, const float *dS_out, const float *dp_out,
                                      float *dq, float *dk, float *dv, float *dlog_alpha,
                                      float *dbeta, float *dproc_noise, float *dobs_noise,
                                      float *dS0, float *dp0, void *workspace,
                                      unsigned long long workspace_bytes, void *stream) {
    int C = 0;
    if (kdn_status st = prefill_shape(variant, dtype, B, T, H, d_k, d_v, chunk, &C))
        return st;
    const bool iso = variant == KDN_ISO_KDN, diag = variant == KDN_DIAG_KDN;
    const bool kdn = iso || diag;
    const long long bh = (long long)B * H;
    const long long tok = bh * T;
    const bool gdn = variant == KDN_GATED_DELTANET, dn = variant == KDN_DELTANET;
    if (tok > 0 && (!q || !k || !v || !d_o || !dq || !dk || !dv))
        return KDN_ERR_NULL;
    if (kdn_status st = check_gates(variant, alpha, beta, proc_noise, obs_noise, tok == 0))
        return st;
    if (dn && dlog_alpha)
        return KDN_ERR_NULL;
    if (!dn && tok > 0 && !dlog_alpha)
        return KDN_ERR_NULL;
    if (kdn) {
        if (dbeta || (bh > 0 && !p0) || (tok > 0 && (!dproc_noise || !dobs_noise)))
            return KDN_ERR_NULL;
    } else {
        if ((tok > 0 && !dbeta) || p0 || dp_out || dproc_noise || dobs_noise || dp0)
            return KDN_ERR_NULL;
    }
    const long long es = dtype == KDN_BF16 ? 2 : 4;
    const void *vec[] = {q, k, v, gdn ? nullptr : alpha, proc_noise, S0, d_o, dS_out, dq, dk,
                         dv, gdn ? nullptr : dlog_alpha, dproc_noise, dS0,
                         diag ? (const void *)p0 : nullptr, diag ? (const void *)dp_out : nullptr,
                         diag ? (const void *)dp0 : nullptr};
    for (const void *x : vec)
        if (x && !aligned(x, 16))
            return KDN_ERR_ALIGN;
    for (const void *x : {beta, obs_noise, gdn ? alpha : nullptr})
        if (x && !aligned(x, (uintptr_t)es))
            return KDN_ERR_ALIGN;
    for (const void *x : {(const void *)dbeta, (const void *)(gdn ? dlog_alpha : nullptr),
                          (const void *)dobs_noise, (const void *)p0, (const void *)dp_out,
                          (const void *)dp0})
        if (x && !aligned(x, 4))
            return KDN_ERR_ALIGN;

    const long long n_qk = tok * d_k * es, n_v = tok * d_v * es;
    const long long n_a = gdn ? tok * es : (dn ? 0 : tok * d_k * es);
    const long long n_S = bh * d_k * d_v * 4;
    const long long n_p = bh * p_per_head(variant, d_k) * 4;
    struct R { const void *p; long long n; };
    const R ins[] = {{q, n_qk}, {k, n_qk}, {v, n_v}, {alpha, n_a}, {beta, kdn ? 0 : tok * es},
                     {proc_noise, kdn ? n_qk : 0}, {obs_noise, kdn ? tok * es : 0},
                     {S0, n_S}, {p0, n_p}, {d_o, n_v}, {dS_out, n_S}, {dp_out, n_p}};
    const R outs[] = {{dq, tok * d_k * 4}, {dk, tok * d_k * 4}, {dv, tok * d_v * 4},
                      {dlog_alpha, gdn ? tok * 4 : (dn ? 0 : tok * d_k * 4)},
                      {dbeta, kdn ? 0 : tok * 4}, {dproc_noise, kdn ? tok * d_k * 4 : 0},
                      {dobs_noise, kdn ? tok * 4 : 0}, {dS0, n_S}, {dp0, n_p}};
    constexpr int NO = (int)(sizeof(outs) / sizeof(outs[0]));
    // outputs overlap no input and no other output
    for (int i = 0; i < NO; ++i) {
        for (const R &x : ins)
            if (overlap(outs[i].p, outs[i].n, x.p, x.n)) return KDN_ERR_ALIAS;
        for (int j = i + 1; j < NO; ++j)
            if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return KDN_ERR_ALIAS;
    }
    const BwdWs W = backward_ws(variant, dtype == KDN_BF16, B, T, H, d_k, d_v, C);
    if (W.total > 0) {
        if (!workspace || (long long)workspace_bytes < W.total)
            return KDN_ERR_WORKSPACE;
        if (!aligned(workspace, 256))
            return KDN_ERR_ALIGN;
        for (const R &x : ins)
            if (overlap(workspace, W.total, x.p, x.n)) return KDN_ERR_ALIAS;
        for (const R &x : outs)
            if (overlap(workspace, W.total, x.p, x.n)) return KDN_ERR_ALIAS;
    }
    if (bh == 0)
        return KDN_OK;

    // forward: records (isotropic KDN: its variance pass first), then S at
    // every chunk start
    const long long nc = kdn::num_chunks(T, C);
    char *base = static_cast<char *>(workspace);
    kdn::PrefillParams F;
    F.variant = variant;
    F.bf16 = dtype == KDN_BF16;
    F.B = B; F.T = T; F.H = H; F.dk = d_k; F.dv = d_v; F.chunk = C;
    F.mu = mu;
    F.q = q; F.k = k; F.v = v; F.alpha = alpha; F.beta = iso ? nullptr : beta;
    F.xi = proc_noise; F.r = obs_noise;
    F.S0 = S0; F.p0 = p0; F.o = nullptr; F.S_out = nullptr; F.p_out = nullptr;
    F.ws = nullptr; F.ws_mob = nullptr; F.ws_p0 = nullptr; F.ws_pre = nullptr;
    F.ws_stat = nullptr;
    // bf16: records in the permuted order of the chain kernel, which re-runs
    // the forward and saves S at every chunk start; the gradient kernels
    // restore the order when they stage the records
    F.rec_perm = dtype == KDN_BF16 ? 1 : 0;
    F.states = nullptr; F.beta_out = nullptr; F.w_out = nullptr; F.invs_out = nullptr;
    F.cus = device_cus();
    if (W.total > 0) {
        F.ws = base;
        F.states = base + W.states;
        if (iso) {
            char *vb = base + kdn::WsLayout::make(dtype == KDN_BF16, C, d_k).records(bh, nc);
            const long long n_mob = kdn::WsLayout::mobius_bytes(bh, nc, 1);
            F.ws_mob = reinterpret_cast<float *>(vb);
            F.ws_stat = reinterpret_cast<float *>(vb + n_mob);
            F.ws_p0 = reinterpret_cast<float *>(vb + n_mob + kdn::WsLayout::stat_bytes(bh, nc, C));
            F.beta_out = reinterpret_cast<float *>(base + W.beta);
        }
        if (diag) {
            char *vb = base + kdn::WsLayout::make(dtype == KDN_BF16, C, d_k).records(bh, nc);
            const long long n_mob = kdn::WsLayout::mobius_bytes(bh, nc, d_k);
            F.ws_mob = reinterpret_cast<float *>(vb);
            F.ws_p0 = reinterpret_cast<float *>(vb + n_mob);
            F.ws_pre = reinterpret_cast<float *>(vb + n_mob +
                                                 kdn::WsLayout::p0_bytes(bh, nc, d_k));
            F.w_out = reinterpret_cast<float *>(base + W.w);
            F.invs_out = reinterpret_cast<float *>(base + W.invs);
        }
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (tok > 0) {
        if (kdn)
            e = kdn::launch_variance_scan(F, st);
        if (e == hipSuccess) {
            switch (variant) {
            case KDN_DELTANET: e = kdn::launch_prefill_prep_v0(F, st); break;
            case KDN_GATED_DELTANET: e = kdn::launch_prefill_prep_v1(F, st); break;
            case KDN_KDA: e = kdn::launch_prefill_prep_v2(F, st); break;
            case KDN_DIAG_KDN: e = kdn::launch_prefill_prep_v3(F, st); break;
            default: e = kdn::launch_prefill_prep_v4(F, st); break;
            }
        }
        if (e == hipSuccess)
            e = F.rec_perm ? kdn::launch_prefill_chain(F, st) : kdn::launch_prefill_state(F, st);
        if (e != hipSuccess)
            return KDN_ERR_HIP;
    }
    kdn::BackwardParams G;
    G.variant = variant;
    G.bf16 = dtype == KDN_BF16;
    G.B = B; G.T = T; G.H = H; G.dk = d_k; G.dv = d_v; G.chunk = C;
    G.mu = mu;
    G.q = q; G.k = k; G.v = v; G.alpha = alpha; G.beta = kdn ? nullptr : beta;
    G.xi = proc_noise; G.r = obs_noise; G.p0 = p0;
    G.beta_f32 = F.beta_out;
    G.w_f32 = F.w_out;
    const bool dws = diag && W.total > 0;
    G.dw_out = dws ? reinterpret_cast<float *>(base + W.dw) : nullptr;
    G.invs = F.invs_out;
    G.wdw = dws ? reinterpret_cast<float *>(base + W.wdw) : nullptr;
    G.pp = dws ? reinterpret_cast<float *>(base + W.pp) : nullptr;
    G.S0 = S0;
    G.dO = d_o; G.dS_out = dS_out;
    G.dq = dq; G.dk_ = dk; G.dv_ = dv; G.dla = dlog_alpha;
    G.dbeta = iso ? (W.total > 0 ? reinterpret_cast<float *>(base + W.dbeta) : nullptr)
                  : (diag ? nullptr : dbeta);
    G.dS0 = dS0;
    G.dp_out = dp_out; G.dxi = dproc_noise; G.dr = dobs_noise; G.dp0 = dp0;
    G.ws = F.ws;
    G.rec_perm = F.rec_perm;
    G.states = F.states;
    G.dstates = W.total > 0 ? static_cast<void *>(base + W.dstates) : nullptr;
    G.ws_stat = F.ws_stat; G.ws_p0 = F.ws_p0;
    G.chain_map = kdn && W.total > 0 ? reinterpret_cast<float *>(base + W.cmap) : nullptr;
    G.chain_dp = kdn && W.total > 0 ? reinterpret_cast<float *>(base + W.cdp) : nullptr;
    G.cus = F.cus;
    e = kdn::launch_backward(G, st);
    return e == hipSuccess ? KDN_OK : KDN_ERR_HIP;
}

}  // extern "C"
