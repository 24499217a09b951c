// kdn_variance.hip -- KDN variance scans of the two-pass prefill (diagonal
// KDN: one variance per key channel; isotropic KDN: one per head).
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
//      shuffle scan; besides the chunk map it stores the map from the chunk
//      start to the start of each token segment, so the prep kernel can run
//      the per-token chain of all segments of a chunk at once;
//   2. per (batch*head, channel) the chunk maps are composed per segment of
//      chunks, the segment maps applied in order from p0, then each segment's
//      chunk maps from its start: the variance at each chunk start, and p_out.
// Token step with c = mu k^2 / r (r > 0), divided through by r:
//   M = [[a^2, xi], [c a^2, c xi + 1]].
// r = 0: if mu k^2 = 0 the update is the identity (M = [[a^2, xi], [0, 1]]);
// otherwise the update gives 0 for every p- (M = [[0, 0], [0, 1]]).
// All entries are >= 0, so the products have no cancellation; they are
// rescaled every four tokens (the map is unchanged by a common factor).
//
// Isotropic KDN (page "给记忆装一个信任度探测器 ...", section "各向同性近似：把整个头
// 压缩成一个数"): one variance per head, the same step with the channel means
// of a^2 and xi and c = (mu / d_k) |k|^2 / r.  Its chunk kernel also stores
// each token's (mean a^2, mean xi, |k|^2, r), from which the prep kernel
// derives the write strengths without re-reading xi.
#include "kdn_device.h"
#include "kdn_launch.h"
#include "kdn_workspace.h"

namespace kdn {

// Channels per thread: one 16-byte load of k, alpha and xi per token.
template <typename E> struct VarVec { static constexpr int N = 16 / (int)sizeof(E); };

// One wave per (batch*head, chunk): lane = sub * TPU + cg holds channels
// [cg N, cg N + N) over the sub-th of SUBS equal token ranges of the chunk.
// Each lane composes its range (one or two token segments of C / NS tokens,
// NS = WsLayout::var_segments(DK)); an inclusive scan over the ranges (a
// shuffle per level, earlier ranges applied first) gives each lane the map
// from the chunk start to its range end.  The last range's lanes write the
// chunk map; every segment s >= 1 gets the map from the chunk start to its
// first token, from which the prep kernel starts that segment's chain.
template <typename E, int DK>
__global__ __launch_bounds__(256) void variance_chunk_kernel(PrefillParams P) {
    constexpr int N = VarVec<E>::N;                    // channels per lane
    constexpr int TPU = DK / N;                        // lanes per token range
    constexpr int SUBS = WAVE / TPU;                   // token ranges per chunk
    static_assert(TPU * SUBS == WAVE && (SUBS & (SUBS - 1)) == 0, "variance lanes");
    constexpr int NS = WsLayout::var_segments(DK);     // token segments per chunk
    constexpr int Q = NS / SUBS;                       // segments per range
    static_assert(Q * SUBS == NS && (Q == 1 || Q == 2), "variance segments");
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
    const int LG = C / NS;                             // tokens per segment
    const int tb = sub * Q * LG;
    const E *gk = static_cast<const E *>(P.k);
    const E *ga = static_cast<const E *>(P.alpha);
    const E *gx = static_cast<const E *>(P.xi);
    const E *gr = static_cast<const E *>(P.r);
    const float mu = P.mu;

    Map2 m[N];                                         // maps p(range start) -> p
    Map2 h1[N];                                        // Q = 2: over the first segment
#pragma unroll
    for (int e = 0; e < N; ++e)
        m[e] = Map2{1.f, 0.f, 0.f, 1.f};
    const long row0 = ((long)b * T + c0) * H + h;
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        const int te = min(tb + (j + 1) * LG, L);
#pragma unroll 2
        for (int t = tb + j * LG; t < te; ++t) {
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
        if (Q == 2 && j == 0) {
#pragma unroll
            for (int e = 0; e < N; ++e)
                h1[e] = m[e];
        }
    }
    // inclusive scan over the ranges: m <- m o (map of the ranges before)
#pragma unroll
    for (int off = 1; off < SUBS; off <<= 1) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float ya = __shfl_up(m[e].a, off * TPU, WAVE);
            const float yb = __shfl_up(m[e].b, off * TPU, WAVE);
            const float yc = __shfl_up(m[e].c, off * TPU, WAVE);
            const float yd = __shfl_up(m[e].d, off * TPU, WAVE);
            if (sub >= off) {
                m[e].before(ya, yb, yc, yd);
                m[e].rescale();
            }
        }
    }
    const long u = (long)bh * NC + c;
    if (sub == SUBS - 1) {
        float4 *dst = reinterpret_cast<float4 *>(P.ws_mob) + u * DK + i0;
#pragma unroll
        for (int e = 0; e < N; ++e)
            dst[e] = make_float4(m[e].a, m[e].b, m[e].c, m[e].d);
    }
    // segment starts: segment g >= 1 starts from the map over segments
    // 0 .. g-1.  Q = 1: that is the inclusive map of range g - 1, stored by
    // its own lanes.  Q = 2: segment 2 sub starts from the inclusive map of
    // range sub - 1, segment 2 sub + 1 from that map followed by this range's
    // first segment.  Channel i0 + e goes to position e * TPU + i0 / N
    // (pre_pos), so a store instruction writes contiguous entries.
    float4 *pre = reinterpret_cast<float4 *>(P.ws_pre) + u * (NS - 1) * DK + i0 / N;
    if constexpr (Q == 1) {
        if (sub < SUBS - 1) {
#pragma unroll
            for (int e = 0; e < N; ++e)
                pre[(long)sub * DK + e * TPU] = make_float4(m[e].a, m[e].b, m[e].c, m[e].d);
        }
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            Map2 x{__shfl_up(m[e].a, TPU, WAVE), __shfl_up(m[e].b, TPU, WAVE),
                   __shfl_up(m[e].c, TPU, WAVE), __shfl_up(m[e].d, TPU, WAVE)};
            if (sub == 0)
                x = Map2{1.f, 0.f, 0.f, 1.f};
            if (sub > 0)
                pre[(long)(2 * sub - 1) * DK + e * TPU] = make_float4(x.a, x.b, x.c, x.d);
            x.after(h1[e].a, h1[e].b, h1[e].c, h1[e].d);
            x.rescale();
            pre[(long)(2 * sub) * DK + e * TPU] = make_float4(x.a, x.b, x.c, x.d);
        }
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
        if (P.p_out)                                   // not kept by the gradient pass
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

// Isotropic KDN, one wave per (batch*head, chunk), chunk-major like the
// diagonal kernel: lane = sub * TPU + g reads channels [g N, g N + N) of the
// tokens of the sub-th token range; the per-token channel sums are combined
// across the TPU lanes of a range by a butterfly, every lane of the range
// composes the token maps, and the ranges are combined in a shuffle tree.
template <typename E, int DK>
__global__ __launch_bounds__(256) void iso_variance_chunk_kernel(PrefillParams P) {
    constexpr int N = VarVec<E>::N;
    constexpr int TPU = DK / N;
    constexpr int SUBS = WAVE / TPU;
    static_assert(TPU * SUBS == WAVE && (SUBS & (SUBS - 1)) == 0, "variance lanes");
    const int C = P.chunk, T = P.T, H = P.H;
    const int NC = (T + C - 1) / C;
    const long unit = (long)blockIdx.x * (256 / WAVE) + threadIdx.x / WAVE;
    if (unit >= (long)P.B * H * NC)                    // whole waves
        return;
    const int lane = threadIdx.x & (WAVE - 1);
    const int sub = lane / TPU, g = lane % TPU, i0 = g * N;
    const long BH = (long)P.B * H;
    const int bh = (int)(unit % BH), c = (int)(unit / BH);
    const int b = bh / H, h = bh % H;
    const int c0 = c * C, L = min(C, T - c0);
    const int LS = C / SUBS;
    const int tb = sub * LS, te = min(tb + LS, L);
    const E *gk = static_cast<const E *>(P.k);
    const E *ga = static_cast<const E *>(P.alpha);
    const E *gx = static_cast<const E *>(P.xi);
    const E *gr = static_cast<const E *>(P.r);
    const float mdk = P.mu * (1.f / DK);
    float4 *stat = reinterpret_cast<float4 *>(P.ws_stat) + ((long)bh * NC + c) * C;

    Map2 m{1.f, 0.f, 0.f, 1.f};
    const long row0 = ((long)b * T + c0) * H + h;
#pragma unroll 2
    for (int t = tb; t < te; ++t) {
        const long row = row0 + (long)t * H;
        float k[N], a[N], x[N];
        load16(gk + row * DK + i0, k);
        load16(ga + row * DK + i0, a);
        load16(gx + row * DK + i0, x);
        const float r = to_f32(gr[row]);
        float sa = 0.f, sx = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            sa = fmaf(a[e], a[e], sa);
            sx += x[e];
            sk = fmaf(k[e], k[e], sk);
        }
#pragma unroll
        for (int off = TPU / 2; off >= 1; off >>= 1) {
            sa += __shfl_xor(sa, off, WAVE);
            sx += __shfl_xor(sx, off, WAVE);
            sk += __shfl_xor(sk, off, WAVE);
        }
        const float a2 = sa * (1.f / DK), xm = sx * (1.f / DK);
        if (g == 0)
            stat[t] = make_float4(a2, xm, sk, r);
        const Map2 y = variance_step_map(a2, xm, mdk * sk, r);
        m.after(y.a, y.b, y.c, y.d);
        if (((t - tb) & 3) == 3)
            m.rescale();
    }
#pragma unroll
    for (int off = 1; off < SUBS; off <<= 1) {
        const bool take = (sub & (2 * off - 1)) == 0;
        const float ya = __shfl_down(m.a, off * TPU, WAVE);
        const float yb = __shfl_down(m.b, off * TPU, WAVE);
        const float yc = __shfl_down(m.c, off * TPU, WAVE);
        const float yd = __shfl_down(m.d, off * TPU, WAVE);
        if (take) {
            m.after(ya, yb, yc, yd);
            m.rescale();
        }
    }
    if (lane == 0)
        reinterpret_cast<float4 *>(P.ws_mob)[(long)bh * NC + c] =
            make_float4(m.a, m.b, m.c, m.d);
}

// Isotropic KDN, one wave per batch*head: lane = segment of LEN chunks.  Each
// lane composes its segment's chunk maps, an inclusive scan over the lanes
// gives the map from p0 to every segment end, and each lane then applies its
// chunk maps from its segment start, storing the variance at every chunk
// start.  Dependent chain: LEN + 6 + LEN steps instead of NC.
__global__ __launch_bounds__(WAVE) void iso_variance_scan_kernel(PrefillParams P) {
    const int NC = (P.T + P.chunk - 1) / P.chunk;
    const long bh = blockIdx.x;
    const int lane = threadIdx.x;
    const int LEN = (NC + WAVE - 1) / WAVE;
    const int cb = min(lane * LEN, NC), ce = min(cb + LEN, NC);
    const float4 *mob = reinterpret_cast<const float4 *>(P.ws_mob) + bh * NC;
    float *ps = P.ws_p0 + bh * NC;

    Map2 m{1.f, 0.f, 0.f, 1.f};
    for (int c = cb; c < ce; ++c) {
        const float4 y = mob[c];
        m.after(y.x, y.y, y.z, y.w);
        if (((c - cb) & 3) == 3)
            m.rescale();
    }
    m.rescale();
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const float ya = __shfl_up(m.a, off, WAVE), yb = __shfl_up(m.b, off, WAVE);
        const float yc = __shfl_up(m.c, off, WAVE), yd = __shfl_up(m.d, off, WAVE);
        if (lane >= off) {
            m.before(ya, yb, yc, yd);
            m.rescale();
        }
    }
    const float p0 = P.p0[bh];
    const float pe = m.apply(p0);                      // variance at segment end
    float p = __shfl_up(pe, 1, WAVE);
    if (lane == 0)
        p = p0;
    if (lane == WAVE - 1 && P.p_out)                   // not kept by the gradient pass
        P.p_out[bh] = pe;
    for (int c = cb; c < ce; ++c) {
        const float4 y = mob[c];
        ps[c] = p;
        p = fmaf(y.x, p, y.y) / fmaf(y.z, p, y.w);
    }
}

template <typename E, int DK>
static hipError_t launch_iso_dk(const PrefillParams &P, hipStream_t st) {
    const long bh = (long)P.B * P.H;
    const long nc = (P.T + P.chunk - 1) / P.chunk;
    if (nc > 0) {
        constexpr int UPW = 256 / WAVE;
        const dim3 grid((unsigned)((bh * nc + UPW - 1) / UPW)), block(256);
        hipLaunchKernelGGL((iso_variance_chunk_kernel<E, DK>), grid, block, 0, st, P);
        if (hipError_t e = hipGetLastError())
            return e;
    }
    const dim3 grid((unsigned)bh), block(WAVE);
    hipLaunchKernelGGL(iso_variance_scan_kernel, grid, block, 0, st, P);
    return hipGetLastError();
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
    if (P.variant == ISO_KDN) {
        if (P.dk == 128)
            return P.bf16 ? launch_iso_dk<bf16, 128>(P, st) : launch_iso_dk<float, 128>(P, st);
        if (P.dk == 64)
            return P.bf16 ? launch_iso_dk<bf16, 64>(P, st) : launch_iso_dk<float, 64>(P, st);
        return hipErrorInvalidValue;
    }
    if (P.dk == 128)
        return P.bf16 ? launch_variance_dk<bf16, 128>(P, st) : launch_variance_dk<float, 128>(P, st);
    if (P.dk == 64)
        return P.bf16 ? launch_variance_dk<bf16, 64>(P, st) : launch_variance_dk<float, 64>(P, st);
    return hipErrorInvalidValue;
}

}  // namespace kdn
