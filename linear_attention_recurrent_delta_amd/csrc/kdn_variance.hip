// kdn_variance.hip -- diagonal-KDN variance scan of the two-pass prefill.
//
// Per key channel the variance follows a scalar recurrence that does not
// involve S or the other channels (predict p- = a^2 p + xi, then the
// mean-field update p = p- r / (r + mu p- k^2)).  Both steps are linear
// fractional maps of p, so each token's step is a 2 x 2 matrix acting on
// (p, 1) projectively and a run of tokens composes by matrix products
// ("给记忆装一个信任度探测器 ...", section "对角近似：把矩阵压扁成一个向量":
// channels evolve independently and the update has Mobius form, which gives
// a parallel scan).  The two kernels here give the prep kernel the variance
// at the start of every chunk without a sequential pass over all tokens:
//   1. one thread per (batch*head, chunk, channel) composes the chunk's maps;
//   2. one thread per (batch*head, channel) applies the chunk maps in order,
//      storing the variance at each chunk start, and p_out at the end.
// Token step with c = mu k^2 / r (r > 0), divided through by r:
//   M = [[a^2, xi], [c a^2, c xi + 1]].
// r = 0: if mu k^2 = 0 the update is the identity (M = [[a^2, xi], [0, 1]]);
// otherwise the update gives 0 for every p- (M = [[0, 0], [0, 1]]).
// All entries are >= 0, so the products have no cancellation; they are
// rescaled every four tokens (the map is unchanged by a common factor).
#include "kdn_device.h"
#include "kdn_launch.h"
#include "kdn_workspace.h"

namespace kdn {

// Channels per thread: one 16-byte load of k, alpha and xi per token.
template <typename E> struct VarVec { static constexpr int N = 16 / (int)sizeof(E); };

template <typename E, int DK>
__global__ __launch_bounds__(256) void variance_chunk_kernel(PrefillParams P) {
    constexpr int N = VarVec<E>::N;                    // channels per thread
    constexpr int TPU = DK / N;                        // threads per (head, chunk)
    constexpr int UPW = 256 / TPU;                     // units per workgroup
    const int C = P.chunk, T = P.T, H = P.H;
    const int NC = (T + C - 1) / C;
    const long unit = (long)blockIdx.x * UPW + threadIdx.x / TPU;
    const int i0 = (threadIdx.x % TPU) * N;
    if (unit >= (long)P.B * H * NC)
        return;
    const int bh = (int)(unit / NC), c = (int)(unit % NC);
    const int b = bh / H, h = bh % H;
    const int c0 = c * C, L = min(C, T - c0);
    const E *gk = static_cast<const E *>(P.k);
    const E *ga = static_cast<const E *>(P.alpha);
    const E *gx = static_cast<const E *>(P.xi);
    const E *gr = static_cast<const E *>(P.r);
    const float mu = P.mu;

    float m00[N], m01[N], m10[N], m11[N];              // maps p(chunk start) -> p
#pragma unroll
    for (int e = 0; e < N; ++e) {
        m00[e] = 1.f; m01[e] = 0.f; m10[e] = 0.f; m11[e] = 1.f;
    }
    const long row0 = ((long)b * T + c0) * H + h;
#pragma unroll 2
    for (int t = 0; t < L; ++t) {
        const long row = row0 + (long)t * H;
        float k[N], a[N], x[N];
        load16(gk + row * DK + i0, k);
        load16(ga + row * DK + i0, a);
        load16(gx + row * DK + i0, x);
        const float r = to_f32(gr[row]);
        const float rinv = r > 0.f ? 1.f / r : 0.f;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float a2 = a[e] * a[e], mk2 = mu * k[e] * k[e];
            float n00 = a2, n01 = x[e], n10 = 0.f, n11 = 1.f;
            if (r > 0.f) {
                const float cc = mk2 * rinv;
                n10 = cc * a2;
                n11 = fmaf(cc, x[e], 1.f);
            } else if (mk2 != 0.f) {
                n00 = 0.f;
                n01 = 0.f;
            }
            const float p00 = n00 * m00[e] + n01 * m10[e], p01 = n00 * m01[e] + n01 * m11[e];
            const float p10 = n10 * m00[e] + n11 * m10[e], p11 = n10 * m01[e] + n11 * m11[e];
            m00[e] = p00; m01[e] = p01; m10[e] = p10; m11[e] = p11;
            if ((t & 3) == 3) {
                const float sc = fast_rcp(fmaxf(fmaxf(m00[e], m01[e]), fmaxf(m10[e], m11[e])));
                m00[e] *= sc; m01[e] *= sc; m10[e] *= sc; m11[e] *= sc;
            }
        }
    }
    float4 *dst = reinterpret_cast<float4 *>(P.ws_mob) + unit * DK + i0;
#pragma unroll
    for (int e = 0; e < N; ++e)
        dst[e] = make_float4(m00[e], m01[e], m10[e], m11[e]);
}

template <int DK>
__global__ __launch_bounds__(64) void variance_scan_kernel(PrefillParams P) {
    const long g = (long)blockIdx.x * 64 + threadIdx.x;     // (bh, channel)
    if (g >= (long)P.B * P.H * DK)
        return;
    const long bh = g / DK;
    const int i = (int)(g % DK);
    const int NC = (P.T + P.chunk - 1) / P.chunk;
    const float4 *mob = reinterpret_cast<const float4 *>(P.ws_mob) + bh * NC * DK + i;
    float *p0 = P.ws_p0 + bh * NC * DK + i;
    float p = P.p0[g];
    int c = 0;
    for (; c + 4 <= NC; c += 4) {                  // maps read ahead of the chain
        float4 m[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            m[u] = mob[(long)(c + u) * DK];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            p0[(long)(c + u) * DK] = p;
            p = fmaf(m[u].x, p, m[u].y) / fmaf(m[u].z, p, m[u].w);
        }
    }
    for (; c < NC; ++c) {
        const float4 m = mob[(long)c * DK];
        p0[(long)c * DK] = p;
        p = fmaf(m.x, p, m.y) / fmaf(m.z, p, m.w);
    }
    P.p_out[g] = p;
}

template <typename E, int DK>
static hipError_t launch_variance_dk(const PrefillParams &P, hipStream_t st) {
    const long bh = (long)P.B * P.H;
    const long nc = (P.T + P.chunk - 1) / P.chunk;
    if (nc > 0) {
        constexpr int UPW = 256 / (DK / VarVec<E>::N);
        const dim3 grid((unsigned)((bh * nc + UPW - 1) / UPW)), block(256);
        hipLaunchKernelGGL((variance_chunk_kernel<E, DK>), grid, block, 0, st, P);
        if (hipError_t e = hipGetLastError())
            return e;
    }
    const dim3 grid((unsigned)((bh * DK + 63) / 64)), block(64);
    hipLaunchKernelGGL((variance_scan_kernel<DK>), grid, block, 0, st, P);
    return hipGetLastError();
}

hipError_t launch_variance_scan(const PrefillParams &P, hipStream_t st) {
    if (P.dk == 128)
        return P.bf16 ? launch_variance_dk<bf16, 128>(P, st) : launch_variance_dk<float, 128>(P, st);
    if (P.dk == 64)
        return P.bf16 ? launch_variance_dk<bf16, 64>(P, st) : launch_variance_dk<float, 64>(P, st);
    return hipErrorInvalidValue;
}

}  // namespace kdn
