// kdn_decode.hip -- fused single-token decode step (gfx950).
//
// One workgroup of 256 threads owns one (sequence, head) memory S (d_k x d_v
// float32) and reads and writes it exactly once per step; the step is bound
// by HBM traffic on S.  This is the fused-recurrent regime of the page
// "معماری KDA: حذف تداخل حافظه با قانون دلتا در توالی‌های بلند", section
// "پیاده‌سازی فنی و گذارهای DPLR" (token-by-token vector work for decode).
//
// Per token (page "Внимание в LLM · часть 11 -- Память с поправкой", section
// "Записать не новое значение, а ошибку памяти"; decay first, section "از
// فراموشی کلی به فراموشی جزئی" of the KDA page):
//   S- = diag(a) S,  e = v - S-^T k,  S = S- + w e^T,  o = S^T q.
// Diagonal KDN write vector (page "给记忆装一个信任度探测器：Kalman Delta Networks
// 如何让AI知道自己"记得准不准"", sections "把记忆问题重新想成一个滤波问题" and
// "对角近似：把矩阵压扁成一个向量"):
//   p- = a*a*p + xi,  s = r + sum_i p-_i k_i^2,  w = p- k / s,
//   p_i = p-_i r / (r + mu p-_i k_i^2).
// Isotropic KDN (same page, section "各向同性近似：把整个头压缩成一个数"), one
// variance p per head:
//   p- = mean(a^2) p + mean(xi),  w = p- k / (r + p- |k|^2),
//   p = p- r / (r + (mu / d_k) p- |k|^2).
//
// Thread layout: the d_v columns are split in groups of 4 (one float4 per
// row), the d_k rows in RG groups; thread (rg, cg) holds rows
// [rg*RPT, rg*RPT + RPT) of columns [4 cg, 4 cg + 4) in registers.  A row is
// d_v * 4 contiguous bytes, so 32 consecutive threads stream 512 B.
#include "kdn_device.h"
#include "kdn_launch.h"

namespace kdn {

#ifndef KDN_DECODE_NT
#define KDN_DECODE_NT 256
#endif

// Per-token inputs of one head: the d_k vectors (k, q, decay, process noise)
// in threads < d_k, the per-head scalars, and this thread's 4 values of v.
template <typename TIn, int VAR, int DK>
struct TokenIn {
    float k = 0.f, q = 0.f, a = 1.f, xi = 0.f, beta = 0.f, r = 0.f;
    float v[4] = {0.f, 0.f, 0.f, 0.f};

    __device__ __forceinline__ void load(const DecodeParams &P, long row, int tid, int cg) {
        if (tid < DK) {
            k = to_f32(static_cast<const TIn *>(P.k)[row * DK + tid]);
            q = to_f32(static_cast<const TIn *>(P.q)[row * DK + tid]);
            if (VAR == GATED_DELTANET)
                a = to_f32(static_cast<const TIn *>(P.alpha)[row]);
            else if (VAR == KDA || VAR == DIAG_KDN || VAR == ISO_KDN)
                a = to_f32(static_cast<const TIn *>(P.alpha)[row * DK + tid]);
            if (VAR == DIAG_KDN || VAR == ISO_KDN)
                xi = to_f32(static_cast<const TIn *>(P.xi)[row * DK + tid]);
            else
                beta = to_f32(static_cast<const TIn *>(P.beta)[row]);
        }
        if (VAR == DIAG_KDN || VAR == ISO_KDN)
            r = to_f32(static_cast<const TIn *>(P.r)[row]);
        const TIn *vp = static_cast<const TIn *>(P.v) + row * P.dv + 4 * cg;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = to_f32(vp[e]);
    }
};

// MULTI = false: one token per (sequence, head), S and p updated in place
// (P.S0 == P.S, P.p0 == P.p).  MULTI = true: P.T tokens per (sequence, head)
// with per-token tensors [N, T, H, .]; S and p are read from S0 / p0 once,
// stepped through the T tokens in registers, and written to S / p once.  The
// arithmetic of a token is the same in both.
template <typename TIn, int VAR, int DK, int DV, int NT, bool MULTI>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeParams P) {
    constexpr int CG = DV / 4;        // float4 column groups
    constexpr int RG = NT / CG;       // row groups
    constexpr int RPT = DK / RG;      // rows per thread
    static_assert(RPT * RG == DK && CG * RG == NT, "decode tiling");

    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const long bh = blockIdx.x;
    const int T = MULTI ? P.T : 1;
    // row of token t in the per-token tensors: (n, t, h) for [N, T, H, .]
    const long n = MULTI ? bh / P.H : 0, h = MULTI ? bh % P.H : bh;
    auto row_of = [&](int t) { return MULTI ? (n * T + t) * P.H + h : bh; };

    const float *Sin = P.S0 ? P.S0 + bh * (long)DK * DV : nullptr;
    float *S = P.S + bh * (long)DK * DV;
    const int row0 = rg * RPT;

    __shared__ float sk[DK], sq[DK], sa[DK], sg[DK];
    // partial column sums of the read (red) and of the output (ored): two
    // buffers, so no barrier separates reading one from writing the other
    __shared__ f32x4 red[RG][CG], ored[RG][CG];
    __shared__ float part[3][NT / WAVE];

    // The first token's vectors are requested first and the state after
    // them: loads return in order, so the gain below is formed while the
    // state is still streaming in.
    TokenIn<TIn, VAR, DK> in;
    if (T > 0)
        in.load(P, row_of(0), tid, cg);
    float pc = 0.f;                   // variance of channel tid (diagonal KDN),
                                      // of the head (isotropic KDN)
    if (VAR == DIAG_KDN && tid < DK)
        pc = P.p0[bh * DK + tid];
    if (VAR == ISO_KDN)
        pc = P.p0[bh];
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = Sin ? __builtin_nontemporal_load(
                         reinterpret_cast<const f32x4 *>(Sin + (long)(row0 + m) * DV) + cg)
                   : f32x4{0.f, 0.f, 0.f, 0.f};

    for (int t = 0; t < T; ++t) {
        TokenIn<TIn, VAR, DK> nxt;    // next token's inputs, in flight meanwhile
        if (MULTI && t + 1 < T)
            nxt.load(P, row_of(t + 1), tid, cg);

        float pm = 0.f, u = 0.f, pk2 = 0.f;
        if (tid < DK) {
            sk[tid] = in.k;
            sq[tid] = in.q;
            sa[tid] = in.a;
            if (VAR == DIAG_KDN) {
                pm = in.a * in.a * pc + in.xi;          // predict
                u = pm * in.k;
                pk2 = u * in.k;
            } else if (VAR != ISO_KDN) {
                sg[tid] = in.beta * in.k;
            }
        }
        if (VAR == ISO_KDN) {
            // channel sums of a^2, xi and k^2 (block reduction), then the
            // scalar predict, gain and update in every thread < DK
            const bool ch = tid < DK;
            const float wa = wave_sum(ch ? in.a * in.a : 0.f);
            const float wx = wave_sum(ch ? in.xi : 0.f);
            const float wk = wave_sum(ch ? in.k * in.k : 0.f);
            if ((tid & (WAVE - 1)) == 0) {
                part[0][tid / WAVE] = wa;
                part[1][tid / WAVE] = wx;
                part[2][tid / WAVE] = wk;
            }
            __syncthreads();
            if (ch) {
                float sa = 0.f, sx = 0.f, kk = 0.f;
#pragma unroll
                for (int w = 0; w < (DK + WAVE - 1) / WAVE; ++w) {
                    sa += part[0][w];
                    sx += part[1][w];
                    kk += part[2][w];
                }
                const float r = in.r;
                const float pmi = fmaf(sa * (1.f / DK), pc, sx * (1.f / DK));
                const float s = fmaf(pmi, kk, r);
                sg[tid] = (s != 0.f) ? pmi / s * in.k : 0.f;   // gain
                const float den = fmaf(P.mu * (1.f / DK) * pmi, kk, r);
                pc = (den != 0.f) ? pmi * r / den : pmi;
            }
        }
        if (VAR == DIAG_KDN) {
            // innovation variance s = r + sum_i p-_i k_i^2 (block reduction)
            const float ws = wave_sum(pk2);
            if ((tid & (WAVE - 1)) == 0)
                part[0][tid / WAVE] = ws;
            __syncthreads();
            if (tid < DK) {
                const float r = in.r;
                float sum = r;
#pragma unroll
                for (int w = 0; w < (DK + WAVE - 1) / WAVE; ++w)
                    sum += part[0][w];
                sg[tid] = (sum != 0.f) ? u / sum : 0.f;    // gain
                const float den = r + P.mu * pm * in.k * in.k;
                pc = (den != 0.f) ? pm * r / den : pm;
            }
        }
        __syncthreads();

        // S- = diag(a) S and the partial read over this thread's rows.
        f32x4 vh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float a = sa[row0 + m];
            const float ki = sk[row0 + m];
            s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
            vh.x += s[m].x * ki; vh.y += s[m].y * ki;
            vh.z += s[m].z * ki; vh.w += s[m].w * ki;
        }
        red[rg][cg] = vh;
        __syncthreads();
        float ev[4];
        {
            f32x4 x0 = red[0][cg];
#pragma unroll
            for (int g = 1; g < RG; ++g) {
                const f32x4 x = red[g][cg];
                x0.x += x.x; x0.y += x.y; x0.z += x.z; x0.w += x.w;
            }
            ev[0] = in.v[0] - x0.x;
            ev[1] = in.v[1] - x0.y;
            ev[2] = in.v[2] - x0.z;
            ev[3] = in.v[3] - x0.w;
        }

        // Write S = S- + w e^T, partial output over this thread's rows.
        const bool last = t + 1 == T;
        f32x4 op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float g = sg[row0 + m];
            const float qi = sq[row0 + m];
            s[m].x += g * ev[0]; s[m].y += g * ev[1];
            s[m].z += g * ev[2]; s[m].w += g * ev[3];
            op.x += s[m].x * qi; op.y += s[m].y * qi;
            op.z += s[m].z * qi; op.w += s[m].w * qi;
            if (last)
                __builtin_nontemporal_store(
                    s[m], reinterpret_cast<f32x4 *>(S + (long)(row0 + m) * DV) + cg);
        }
        ored[rg][cg] = op;
        __syncthreads();
        if (tid < CG) {
            f32x4 x0 = ored[0][tid];
#pragma unroll
            for (int g = 1; g < RG; ++g) {
                const f32x4 x = ored[g][tid];
                x0.x += x.x; x0.y += x.y; x0.z += x.z; x0.w += x.w;
            }
            TIn *o = static_cast<TIn *>(P.o) + row_of(t) * DV + 4 * tid;
            o[0] = from_f32<TIn>(x0.x);
            o[1] = from_f32<TIn>(x0.y);
            o[2] = from_f32<TIn>(x0.z);
            o[3] = from_f32<TIn>(x0.w);
        }
        if (MULTI)
            in = nxt;
    }
    if (MULTI && T == 0) {             // no token: the state passes through
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            __builtin_nontemporal_store(
                s[m], reinterpret_cast<f32x4 *>(S + (long)(row0 + m) * DV) + cg);
    }
    if (VAR == DIAG_KDN && tid < DK)
        P.p[bh * DK + tid] = pc;
    if (VAR == ISO_KDN && tid == 0)
        P.p[bh] = pc;
}

template <typename TIn, int VAR, bool MULTI>
static hipError_t launch_decode_v(const DecodeParams &P, hipStream_t st) {
    constexpr int NT = KDN_DECODE_NT;
    const dim3 grid((unsigned)((long)P.N * P.H)), block(NT);
#define KDN_DEC(DK_, DV_)                                                      \
    if (P.dk == DK_ && P.dv == DV_) {                                          \
        hipLaunchKernelGGL((decode_kernel<TIn, VAR, DK_, DV_, NT, MULTI>), grid, \
                           block, 0, st, P);                                   \
        return hipGetLastError();                                              \
    }
    KDN_DEC(64, 64)
    KDN_DEC(64, 128)
    KDN_DEC(128, 64)
    KDN_DEC(128, 128)
#undef KDN_DEC
    return hipErrorInvalidValue;
}

template <typename TIn, bool MULTI>
static hipError_t launch_decode_t(const DecodeParams &P, hipStream_t st) {
    switch (P.variant) {
    case DELTANET: return launch_decode_v<TIn, DELTANET, MULTI>(P, st);
    case GATED_DELTANET: return launch_decode_v<TIn, GATED_DELTANET, MULTI>(P, st);
    case KDA: return launch_decode_v<TIn, KDA, MULTI>(P, st);
    case DIAG_KDN: return launch_decode_v<TIn, DIAG_KDN, MULTI>(P, st);
    case ISO_KDN: return launch_decode_v<TIn, ISO_KDN, MULTI>(P, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams &P, hipStream_t st) {
    if ((long)P.N * P.H == 0)
        return hipSuccess;
    return P.bf16 ? launch_decode_t<bf16, false>(P, st) : launch_decode_t<float, false>(P, st);
}

hipError_t launch_decode_multi(const DecodeParams &P, hipStream_t st) {
    if ((long)P.N * P.H == 0)
        return hipSuccess;
    return P.bf16 ? launch_decode_t<bf16, true>(P, st) : launch_decode_t<float, true>(P, st);
}

}  // namespace kdn
