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
//   1. one wave per (batch*head, chunk) composes the chunk's maps, each lane
//      a range of its tokens for a few channels, the ranges combined in a
//      shuffle tree;
//   2. per (batch*head, channel) the chunk maps are composed per segment of
//      chunks, the segment maps applied in order from p0, then each segment's
//      chunk maps from its start: the variance at each chunk start, and p_out.
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

// 2 x 2 maps, entries >= 0: x <- y x (y applied after x), and a rescale by
// the largest entry (the map is unchanged by a common factor).
struct Map2 {
    float a, b, c, d;     // [[a, b], [c, d]]
    __device__ __forceinline__ void after(float ya, float yb, float yc, float yd) {
        const float na = ya * a + yb * c, nb = ya * b + yb * d;
        const float nc = yc * a + yd * c, nd = yc * b + yd * d;
        a = na; b = nb; c = nc; d = nd;
    }
    __device__ __forceinline__ void rescale() {
        const float sc = fast_rcp(fmaxf(fmaxf(a, b), fmaxf(c, d)));
        a *= sc; b *= sc; c *= sc; d *= sc;
    }
};

// One wave per (batch*head, chunk): lane = sub * TPU + cg holds channels
// [cg N, cg N + N) over the sub-th of SUBS equal token ranges of the chunk.
// Each lane composes its range, then the ranges are combined in a shuffle
// tree (later ranges on the left) and lanes of range 0 write the chunk map.
template <typename E, int DK>
__global__ __launch_bounds__(256) void variance_chunk_kernel(PrefillParams P) {
    constexpr int N = VarVec<E>::N;                    // channels per lane
    constexpr int TPU = DK / N;                        // lanes per token range
    constexpr int SUBS = WAVE / TPU;                   // token ranges per chunk
    static_assert(TPU * SUBS == WAVE && (SUBS & (SUBS - 1)) == 0, "variance lanes");
    const int C = P.chunk, T = P.T, H = P.H;
    const int NC = (T + C - 1) / C;
    const long unit = (long)blockIdx.x * (256 / WAVE) + threadIdx.x / WAVE;
    if (unit >= (long)P.B * H * NC)                    // whole waves
        return;
    const int lane = threadIdx.x & (WAVE - 1);
    const int sub = lane / TPU, i0 = (lane % TPU) * N;
    // chunk-major: neighbouring waves take neighbouring heads of one chunk,
    // whose token rows are adjacent in memory
    const long BH = (long)P.B * H;
    const int bh = (int)(unit % BH), c = (int)(unit / BH);
    const int b = bh / H, h = bh % H;
    const int c0 = c * C, L = min(C, T - c0);
    const int LS = C / SUBS;                           // tokens per range
    const int tb = sub * LS, te = min(tb + LS, L);
    const E *gk = static_cast<const E *>(P.k);
    const E *ga = static_cast<const E *>(P.alpha);
    const E *gx = static_cast<const E *>(P.xi);
    const E *gr = static_cast<const E *>(P.r);
    const float mu = P.mu;

    Map2 m[N];                                         // maps p(range start) -> p
#pragma unroll
    for (int e = 0; e < N; ++e)
        m[e] = Map2{1.f, 0.f, 0.f, 1.f};
    const long row0 = ((long)b * T + c0) * H + h;
#pragma unroll 2
    for (int t = tb; t < te; ++t) {
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
            m[e].after(n00, n01, n10, n11);
            if (((t - tb) & 3) == 3)
                m[e].rescale();
        }
    }
#pragma unroll
    for (int off = 1; off < SUBS; off <<= 1) {
        const bool take = (sub & (2 * off - 1)) == 0;  // then sub + off < SUBS
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float ya = __shfl_down(m[e].a, off * TPU, WAVE);
            const float yb = __shfl_down(m[e].b, off * TPU, WAVE);
            const float yc = __shfl_down(m[e].c, off * TPU, WAVE);
            const float yd = __shfl_down(m[e].d, off * TPU, WAVE);
            if (take) {
                m[e].after(ya, yb, yc, yd);
                m[e].rescale();
            }
        }
    }
    if (sub == 0) {
        float4 *dst = reinterpret_cast<float4 *>(P.ws_mob) + ((long)bh * NC + c) * DK + i0;
#pragma unroll
        for (int e = 0; e < N; ++e)
            dst[e] = make_float4(m[e].a, m[e].b, m[e].c, m[e].d);
    }
}

// One workgroup per (batch*head, 16 channels), thread (seg, ch): the chunks of
// a channel are cut into SEG segments.  Each thread composes its segment's
// chunk maps; one thread per channel then runs the SEG segment maps from p0
// (the variance at every segment start, and p_out); finally each thread
// applies its segment's chunk maps from that start, storing the variance at
// every chunk start.  The dependent chain is SEG + NC / SEG steps long
// instead of NC.
template <int DK>
__global__ __launch_bounds__(256) void variance_scan_kernel(PrefillParams P) {
    constexpr int CH = 16, SEG = 256 / CH;
    static_assert(DK % CH == 0, "channel blocks");
    __shared__ float4 segmap[SEG][CH];
    __shared__ float pstart[SEG][CH];
    const int NC = (P.T + P.chunk - 1) / P.chunk;
    const long bh = blockIdx.x / (DK / CH);
    const int ch = threadIdx.x % CH, seg = threadIdx.x / CH;
    const int i = (int)(blockIdx.x % (DK / CH)) * CH + ch;
    const int LEN = (NC + SEG - 1) / SEG;              // chunks per segment
    const int cb = min(seg * LEN, NC), ce = min(cb + LEN, NC);
    const float4 *mob = reinterpret_cast<const float4 *>(P.ws_mob) + bh * NC * DK + i;
    float *p0 = P.ws_p0 + bh * NC * DK + i;

    Map2 m{1.f, 0.f, 0.f, 1.f};
#pragma unroll 4
    for (int c = cb; c < ce; ++c) {
        const float4 y = mob[(long)c * DK];
        m.after(y.x, y.y, y.z, y.w);
        if (((c - cb) & 3) == 3)
            m.rescale();
    }
    segmap[seg][ch] = make_float4(m.a, m.b, m.c, m.d);
    __syncthreads();
    if (seg == 0) {
        float p = P.p0[bh * DK + i];
#pragma unroll
        for (int s = 0; s < SEG; ++s) {
            pstart[s][ch] = p;
            const float4 y = segmap[s][ch];
            p = fmaf(y.x, p, y.y) / fmaf(y.z, p, y.w);
        }
        P.p_out[bh * DK + i] = p;
    }
    __syncthreads();
    float p = pstart[seg][ch];
#pragma unroll 4
    for (int c = cb; c < ce; ++c) {
        const float4 y = mob[(long)c * DK];
        p0[(long)c * DK] = p;
        p = fmaf(y.x, p, y.y) / fmaf(y.z, p, y.w);
    }
}

template <typename E, int DK>
static hipError_t launch_variance_dk(const PrefillParams &P, hipStream_t st) {
    const long bh = (long)P.B * P.H;
    const long nc = (P.T + P.chunk - 1) / P.chunk;
    if (nc > 0) {
        constexpr int UPW = 256 / WAVE;                // units (waves) per workgroup
        const dim3 grid((unsigned)((bh * nc + UPW - 1) / UPW)), block(256);
        hipLaunchKernelGGL((variance_chunk_kernel<E, DK>), grid, block, 0, st, P);
        if (hipError_t e = hipGetLastError())
            return e;
    }
    const dim3 grid((unsigned)(bh * (DK / 16))), block(256);
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
