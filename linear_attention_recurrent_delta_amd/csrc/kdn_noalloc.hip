// kdn_noalloc.hip -- kdn_chunk_prefill_noalloc: the two-pass chunkwise prefill
// with the library's own static scratch as its workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The scratch is one file-scope device array of KDN_NOALLOC_SCRATCH_BYTES per
// GPU, held by the loaded library until the process ends.  Its device address
// is looked up once per device with hipGetSymbolAddress (the array's name is
// only a host-side stand-in in host code) and cached.  A call whose workspace
// does not fit runs the sequence in segments of whole chunks, batch by batch:
// the recurrence over T1 + T2 tokens equals the recurrence over T2 tokens
// started from the state (S, p) after T1 tokens, so each segment continues
// from the previous one's S_out / p_out in place.  Nothing in the scratch has
// to start at zero (every workspace record is written before it is read).
// Calls that overlap in time on one GPU share its scratch and race.
#include "kdn.h"
#include "kdn_launch.h"
#include "kdn_workspace.h"

#include <atomic>
#include <mutex>

namespace {

__device__ __align__(256) unsigned char scratch[KDN_NOALLOC_SCRATCH_BYTES];

constexpr int MAXDEV = 64;
std::atomic<void *> scratch_ptr[MAXDEV];
std::mutex scratch_mu;

// Device address of this device's scratch (set-up on the device's first call).
void *device_scratch(int dev) {
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess)
            return nullptr;
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" kdn_status kdn_chunk_prefill_noalloc(kdn_variant variant, kdn_dtype dtype, int B,
                                                int T, int H, int d_k, int d_v, int chunk,
                                                float mu, const void *q, const void *k,
                                                const void *v, const void *alpha,
                                                const void *beta, const void *proc_noise,
                                                const void *obs_noise, const float *S0,
                                                const float *p0, void *o, float *S_out,
                                                float *p_out, void *stream) {
    // Every argument of the full call is checked before anything launches.
    int C = 0;
    if (kdn_status st = kdn::prefill_check(variant, dtype, B, T, H, d_k, d_v, chunk, q, k, v,
                                           alpha, beta, proc_noise, obs_noise, S0, p0, o,
                                           S_out, p_out, true, &C))
        return st;
    const unsigned long long need =
        kdn_chunk_prefill_workspace_size(variant, dtype, B, T, H, d_k, d_v, chunk, nullptr);
    if (need == 0)      // no tokens or no heads: nothing uses a workspace
        return kdn_chunk_prefill(variant, dtype, B, T, H, d_k, d_v, chunk, mu, q, k, v, alpha,
                                 beta, proc_noise, obs_noise, S0, p0, o, S_out, p_out, nullptr,
                                 0, stream);
    // Segments of TS tokens (whole chunks) of one sequence at a time, unless
    // the whole call fits.
    const unsigned long long per_chunk =
        kdn_chunk_prefill_workspace_size(variant, dtype, 1, C, H, d_k, d_v, chunk, nullptr);
    const long long chunks = (long long)(KDN_NOALLOC_SCRATCH_BYTES / per_chunk);
    if (chunks < 1)
        return KDN_ERR_SCRATCH;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAXDEV)
        return KDN_ERR_HIP;
    void *ws = device_scratch(dev);
    if (!ws)
        return KDN_ERR_HIP;
    if (need <= KDN_NOALLOC_SCRATCH_BYTES)
        return kdn_chunk_prefill(variant, dtype, B, T, H, d_k, d_v, chunk, mu, q, k, v, alpha,
                                 beta, proc_noise, obs_noise, S0, p0, o, S_out, p_out, ws,
                                 KDN_NOALLOC_SCRATCH_BYTES, stream);
    const long long TS = chunks * C;
    const long long es = dtype == KDN_BF16 ? 2 : 4;
    const long long pph = variant == KDN_DIAG_KDN ? d_k : (variant == KDN_ISO_KDN ? 1 : 0);
    const long long a_w = variant == KDN_GATED_DELTANET ? 1 : (variant == KDN_DELTANET ? 0 : d_k);
    auto off = [](const void *p, long long bytes) -> const void * {
        return p ? static_cast<const char *>(p) + bytes : nullptr;
    };
    kdn_status st = KDN_OK;
    for (int b = 0; b < B; ++b) {
        const float *s_in = S0 ? S0 + (long long)b * H * d_k * d_v : nullptr;
        const float *p_in = p0 ? p0 + (long long)b * H * pph : nullptr;
        float *s_o = S_out + (long long)b * H * d_k * d_v;
        float *p_o = p_out ? p_out + (long long)b * H * pph : nullptr;
        for (long long t0 = 0; t0 < T; t0 += TS) {
            const int tl = (int)(T - t0 < TS ? T - t0 : TS);
            const long long row = ((long long)b * T + t0) * H;   // (b, t0, h = 0)
            st = kdn_chunk_prefill(
                variant, dtype, 1, tl, H, d_k, d_v, chunk, mu, off(q, row * d_k * es),
                off(k, row * d_k * es), off(v, row * d_v * es), off(alpha, row * a_w * es),
                off(beta, row * es), off(proc_noise, row * d_k * es),
                off(obs_noise, row * es), s_in, p_in,
                const_cast<void *>(off(o, row * d_v * es)), s_o, p_o, ws,
                KDN_NOALLOC_SCRATCH_BYTES, stream);
            if (st != KDN_OK)
                return st;
            // later segments continue from this one's state, in place
            s_in = s_o;
            p_in = p_o;
        }
    }
    return KDN_OK;
}

extern "C" unsigned long long kdn_noalloc_scratch_bytes(void) {
    return KDN_NOALLOC_SCRATCH_BYTES;
}
