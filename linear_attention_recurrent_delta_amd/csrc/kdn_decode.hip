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

template <typename TIn, int VAR, int DK, int DV, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeParams P) {
    constexpr int CG = DV / 4;        // float4 column groups
    constexpr int RG = NT / CG;       // row groups
    constexpr int RPT = DK / RG;      // rows per thread
    static_assert(RPT * RG == DK && CG * RG == NT, "decode tiling");

    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const long bh = blockIdx.x;

    float *S = P.S + bh * (long)DK * DV;
    const int row0 = rg * RPT;

    __shared__ float sk[DK], sq[DK], sa[DK], sg[DK];
    __shared__ f32x4 red[RG][CG];
    __shared__ float part[NT / WAVE];

    const TIn *q = static_cast<const TIn *>(P.q) + bh * DK;
    const TIn *k = static_cast<const TIn *>(P.k) + bh * DK;

    // The per-head vectors are requested first and the state after them:
    // loads return in order, so the gain below is formed while the state is
    // still streaming in.
    float kk = 0.f, qq = 0.f, aa = 1.f, xi = 0.f, p0 = 0.f, bt = 0.f;
    if (tid < DK) {
        kk = to_f32(k[tid]);
        qq = to_f32(q[tid]);
        if (VAR == GATED_DELTANET)
            aa = to_f32(static_cast<const TIn *>(P.alpha)[bh]);
        else if (VAR == KDA || VAR == DIAG_KDN)
            aa = to_f32(static_cast<const TIn *>(P.alpha)[bh * DK + tid]);
        if (VAR == DIAG_KDN) {
            xi = to_f32(static_cast<const TIn *>(P.xi)[bh * DK + tid]);
            p0 = P.p[bh * DK + tid];
        } else {
            bt = to_f32(static_cast<const TIn *>(P.beta)[bh]);
        }
    }
    const float rr = VAR == DIAG_KDN ? to_f32(static_cast<const TIn *>(P.r)[bh]) : 0.f;
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(S + (long)(row0 + m) * DV) + cg);

    float pm = 0.f, u = 0.f, pk2 = 0.f;
    if (tid < DK) {
        sk[tid] = kk;
        sq[tid] = qq;
        sa[tid] = aa;
        if (VAR == DIAG_KDN) {
            pm = aa * aa * p0 + xi;                     // predict
            u = pm * kk;
            pk2 = u * kk;
        } else {
            sg[tid] = bt * kk;
        }
    }
    if (VAR == DIAG_KDN) {
        // innovation variance s = r + sum_i p-_i k_i^2 (block reduction)
        const float ws = wave_sum(pk2);
        if ((tid & (WAVE - 1)) == 0)
            part[tid / WAVE] = ws;
        __syncthreads();
        if (tid < DK) {
            const float r = rr;
            float sum = r;
#pragma unroll
            for (int w = 0; w < (DK + WAVE - 1) / WAVE; ++w)
                sum += part[w];
            sg[tid] = (sum != 0.f) ? u / sum : 0.f;    // gain
            const float den = r + P.mu * pm * kk * kk;
            P.p[bh * DK + tid] = (den != 0.f) ? pm * r / den : pm;
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
        f32x4 t = red[0][cg];
#pragma unroll
        for (int g = 1; g < RG; ++g) {
            const f32x4 x = red[g][cg];
            t.x += x.x; t.y += x.y; t.z += x.z; t.w += x.w;
        }
        const TIn *v = static_cast<const TIn *>(P.v) + bh * DV + 4 * cg;
        ev[0] = to_f32(v[0]) - t.x;
        ev[1] = to_f32(v[1]) - t.y;
        ev[2] = to_f32(v[2]) - t.z;
        ev[3] = to_f32(v[3]) - t.w;
    }
    __syncthreads();   // red is reused below

    // Write S = S- + w e^T, partial output over this thread's rows.
    f32x4 op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const float g = sg[row0 + m];
        const float qi = sq[row0 + m];
        s[m].x += g * ev[0]; s[m].y += g * ev[1];
        s[m].z += g * ev[2]; s[m].w += g * ev[3];
        op.x += s[m].x * qi; op.y += s[m].y * qi;
        op.z += s[m].z * qi; op.w += s[m].w * qi;
        __builtin_nontemporal_store(
            s[m], reinterpret_cast<f32x4 *>(S + (long)(row0 + m) * DV) + cg);
    }
    red[rg][cg] = op;
    __syncthreads();
    if (tid < CG) {
        f32x4 t = red[0][tid];
#pragma unroll
        for (int g = 1; g < RG; ++g) {
            const f32x4 x = red[g][tid];
            t.x += x.x; t.y += x.y; t.z += x.z; t.w += x.w;
        }
        TIn *o = static_cast<TIn *>(P.o) + bh * DV + 4 * tid;
        o[0] = from_f32<TIn>(t.x);
        o[1] = from_f32<TIn>(t.y);
        o[2] = from_f32<TIn>(t.z);
        o[3] = from_f32<TIn>(t.w);
    }
}

template <typename TIn, int VAR>
static hipError_t launch_decode_v(const DecodeParams &P, hipStream_t st) {
    constexpr int NT = KDN_DECODE_NT;
    const dim3 grid((unsigned)((long)P.N * P.H)), block(NT);
#define KDN_DEC(DK_, DV_)                                                      \
    if (P.dk == DK_ && P.dv == DV_) {                                          \
        hipLaunchKernelGGL((decode_kernel<TIn, VAR, DK_, DV_, NT>), grid,      \
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

template <typename TIn>
static hipError_t launch_decode_t(const DecodeParams &P, hipStream_t st) {
    switch (P.variant) {
    case DELTANET: return launch_decode_v<TIn, DELTANET>(P, st);
    case GATED_DELTANET: return launch_decode_v<TIn, GATED_DELTANET>(P, st);
    case KDA: return launch_decode_v<TIn, KDA>(P, st);
    case DIAG_KDN: return launch_decode_v<TIn, DIAG_KDN>(P, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams &P, hipStream_t st) {
    if ((long)P.N * P.H == 0)
        return hipSuccess;
    return P.bf16 ? launch_decode_t<bf16>(P, st) : launch_decode_t<float>(P, st);
}

}  // namespace kdn
