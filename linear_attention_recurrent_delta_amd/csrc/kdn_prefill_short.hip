// kdn_prefill_short.hip -- chunkwise prefill of short sequences (gfx950), one
// workgroup per (batch, head), chunks of 16 tokens, bf16 operands.
//
// A few tokens from a resident state -- checking a run of draft tokens of
// speculative decoding is the case in view ("معماری KDA ...", section
// "گام بعدی شما", chunkwise KDA paired with speculative decoding) -- is too
// little work per sequence for the two-pass schedule, whose prep and state
// passes are built for thousands of tokens.  Here one workgroup of four waves
// owns the whole d_k x d_v state of a head in MFMA accumulators (fp32) and
// takes the T <= 16 tokens as one chunk with the chunk algebra of
// kdn_prefill.hip ("حل مشکل وابستگی علی"):
//   E = (I + A_kk)^-1 (V - K~ S),  O = Q~ S + A_qk E,  S <- diag(gamma) S + W~^T E.
// At C = 16 every state product is a 16 x 16 MFMA tile: wave w owns columns
// [w d_v / 4, (w + 1) d_v / 4) of S and computes U, E, O and the S update for
// them; the S-independent part of the chunk (variance chain, decays, scaled
// operands, A_kk, A_qk, the 16 x 16 triangular inverse) is shared through LDS.
//
// Operand layouts (v_mfma_f32_16x16x32_bf16 for contractions over d_k,
// v_mfma_f32_16x16x16_bf16 over the chunk's 16 tokens):
//  - contractions over d_k take S as the B operand straight from the
//    accumulators: lane (q, n) holds rows 4q..4q+3 of two adjacent 16-row
//    tiles, so K~, Q~ and W' are written with the contraction index of each
//    32-group permuted (perm_col in kdn_workspace.h), as the two-pass records
//    are;
//  - contractions over tokens take U and E as the B operand straight from
//    the accumulators: at K = 16 lane (q, n) supplies k = 4q..4q+3, which are
//    the rows it holds, so no permutation is needed.
// The state is read once and written once; the chunk's inputs are requested
// before it, so the S-independent work runs while the state streams in.  That
// work is latency-bound, so three workgroups share a CU (45 KB of LDS and
// under 170 VGPRs per lane each at d_k = 128) and the state traffic of one
// overlaps the chunk work of another.
#include "kdn_device.h"
#include "kdn_launch.h"
#include "kdn_workspace.h"

namespace kdn {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Below this cumulative in-chunk decay the 1/gamma operand scaling is not
// used; the chunk's A matrices take the exact elementwise path.
constexpr float SHORT_DECAY_FLOOR = 8.077935669463161e-28f;   // 2^-90

constexpr int TC = 16;          // tokens per chunk
constexpr int NW = 4;           // waves per workgroup
constexpr int NT = 64 * NW;

template <int DK>
struct ShortLayout {
    static constexpr int PK = DK + 8;          // pitch of the raw [16][DK] tiles
    static constexpr int PU = DK + 4;          // pitch of the fp32 u = p- k tile
    static constexpr int GK = DK / 32;         // 32-groups over d_k
    static constexpr int NIB = DK / 16;        // 16-row blocks of S
    static constexpr int SZ_RAW = TC * PK * 2;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = OFF_K + SZ_RAW;
    static constexpr int OFF_A = OFF_Q + SZ_RAW;
    static constexpr int OFF_X = OFF_A + SZ_RAW;
    static constexpr int OFF_U = OFF_X + SZ_RAW;
    static constexpr int OFF_KF = OFF_U + TC * PU * 4;      // K~ fragments
    static constexpr int OFF_QF = OFF_KF + GK * 64 * 16;    // Q~ fragments
    static constexpr int OFF_WF = OFF_QF + GK * 64 * 16;    // W' fragments
    static constexpr int OFF_WT = OFF_WF + GK * 64 * 16;    // W~^T fragments (K = 16)
    static constexpr int OFF_TF = OFF_WT + NIB * 64 * 8;    // T fragments
    static constexpr int OFF_AQ = OFF_TF + 64 * 8;          // A_qk fragments
    static constexpr int OFF_AKK = OFF_AQ + 64 * 8;         // A_kk, fp32 [16][16]
    static constexpr int OFF_GC = OFF_AKK + TC * TC * 4;    // gamma of the chunk
    static constexpr int OFF_SM = OFF_GC + DK * 4;          // per-token scalars
    static constexpr int SM_R = 0, SM_B = TC, SM_INVS = 2 * TC, SM_A = 3 * TC,
                         SM_IA2 = 4 * TC, SM_IXM = 5 * TC, SM_IKK = 6 * TC,
                         SM_FLAG = 7 * TC;
    static constexpr int TOTAL = OFF_SM + (7 * TC + 4) * 4;
};

__device__ __forceinline__ unsigned short bits(bf16 x) {
    return __builtin_bit_cast(unsigned short, x);
}

// 8 accumulator values (rows 4q..4q+3 of two adjacent 16-row tiles) as the
// bf16 B operand of the permuted k-slots
__device__ __forceinline__ bf16x8 pack8(const f32x4 &lo, const f32x4 &hi) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = static_cast<bf16>(lo[e]);
        r[4 + e] = static_cast<bf16>(hi[e]);
    }
    return r;
}
// 4 accumulator values (rows 4q..4q+3) as the B operand of a K = 16 product
__device__ __forceinline__ s16x4 pack4(const f32x4 &x) {
    s16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        r[e] = (short)bits(static_cast<bf16>(x[e]));
    return r;
}
__device__ __forceinline__ f32x4 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const s16x4 &a, const s16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

}  // namespace

#ifndef KDN_SHORT_WAVES_PER_SIMD
#define KDN_SHORT_WAVES_PER_SIMD 3
#endif

template <int VAR, int DK, int DV>
__global__ __launch_bounds__(NT, KDN_SHORT_WAVES_PER_SIMD) void prefill_short_kernel(PrefillParams P) {
    using LY = ShortLayout<DK>;
    constexpr int PK = LY::PK, PU = LY::PU, GK = LY::GK, NIB = LY::NIB;
    constexpr int NTJ = DV / 64;                 // 16-column tiles per wave
    static_assert(NTJ >= 1 && NTJ * 64 == DV, "four waves of 16-column tiles");
    constexpr bool DECAY = VAR != DELTANET;
    constexpr bool VDECAY = VAR == KDA || VAR == DIAG_KDN || VAR == ISO_KDN;
    constexpr bool KDN = VAR == DIAG_KDN;
    constexpr bool ISO = VAR == ISO_KDN;
    __shared__ __attribute__((aligned(16))) char smem[LY::TOTAL];
    bf16 *Kr = reinterpret_cast<bf16 *>(smem + LY::OFF_K);
    bf16 *Qr = reinterpret_cast<bf16 *>(smem + LY::OFF_Q);
    bf16 *Ar = reinterpret_cast<bf16 *>(smem + LY::OFF_A);
    bf16 *Xr = reinterpret_cast<bf16 *>(smem + LY::OFF_X);
    float *U32 = reinterpret_cast<float *>(smem + LY::OFF_U);
    bf16 *KF = reinterpret_cast<bf16 *>(smem + LY::OFF_KF);
    bf16 *QF = reinterpret_cast<bf16 *>(smem + LY::OFF_QF);
    bf16 *WF = reinterpret_cast<bf16 *>(smem + LY::OFF_WF);
    bf16 *WT = reinterpret_cast<bf16 *>(smem + LY::OFF_WT);
    bf16 *TF = reinterpret_cast<bf16 *>(smem + LY::OFF_TF);
    bf16 *AQ = reinterpret_cast<bf16 *>(smem + LY::OFF_AQ);
    float *Akk = reinterpret_cast<float *>(smem + LY::OFF_AKK);
    float *sgc = reinterpret_cast<float *>(smem + LY::OFF_GC);
    float *sm = reinterpret_cast<float *>(smem + LY::OFF_SM);
    float *s_r = sm + LY::SM_R, *s_b = sm + LY::SM_B, *s_invs = sm + LY::SM_INVS,
          *s_a = sm + LY::SM_A, *s_ia2 = sm + LY::SM_IA2, *s_ixm = sm + LY::SM_IXM,
          *s_ikk = sm + LY::SM_IKK;
    int *s_flag = reinterpret_cast<int *>(sm + LY::SM_FLAG);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, n = lane & 15;
    const int bh = blockIdx.x;
    const int b = bh / P.H, h = bh % P.H;
    const int T = P.T, H = P.H;
    const int c0 = wv * (DV / 4);                 // first column of this wave
    const long hdk = (long)H * DK, hdv = (long)H * DV;   // token strides
    const long seqk = ((long)b * T * H + h) * DK;         // (b, t = 0, h) of q/k/alpha/xi
    const long seqv = ((long)b * T * H + h) * DV;         // of v/o
    const long seqs = (long)b * T * H + h;                // of per-token scalars
    const bf16 *gq = static_cast<const bf16 *>(P.q);
    const bf16 *gk = static_cast<const bf16 *>(P.k);
    const bf16 *gv = static_cast<const bf16 *>(P.v);
    const bf16 *ga = static_cast<const bf16 *>(P.alpha);
    const bf16 *gb = static_cast<const bf16 *>(P.beta);
    const bf16 *gx = static_cast<const bf16 *>(P.xi);
    const bf16 *gr = static_cast<const bf16 *>(P.r);
    bf16 *go = static_cast<bf16 *>(P.o);

    // The chunk's raw tiles, per-token scalars and this wave's v values go
    // to registers first (tokens past the end: k = q = 0, a = 1, xi = 0,
    // r = 1, beta = 0, v = 0 -- no effect on S or p).
    constexpr int TPR = DK / 8;                  // threads per raw row
    const int st_t = tid / TPR, st_c = (tid % TPR) * 8;
    const int L = T;                             // T <= 16: one chunk
    uint4 rk = make_uint4(0u, 0u, 0u, 0u), rq = rk, rx = rk;
    uint4 ra = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
    float rr = 1.f, rb = 0.f, rga = 1.f;
    float rv[NTJ][4];
    if (st_t < L) {
        const long g = seqk + (long)st_t * hdk + st_c;
        rk = *reinterpret_cast<const uint4 *>(gk + g);
        rq = *reinterpret_cast<const uint4 *>(gq + g);
        if (VDECAY)
            ra = *reinterpret_cast<const uint4 *>(ga + g);
        if (KDN || ISO)
            rx = *reinterpret_cast<const uint4 *>(gx + g);
    }
    if (tid < L) {
        const long g = seqs + (long)tid * H;
        if (KDN || ISO)
            rr = to_f32(gr[g]);
        else
            rb = to_f32(gb[g]);
        if (VAR == GATED_DELTANET)
            rga = to_f32(ga[g]);
    }
#pragma unroll
    for (int j = 0; j < NTJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * q + r;
            rv[j][r] = t < L ? to_f32(gv[seqv + (long)t * hdv + c0 + 16 * j + n]) : 0.f;
        }

    // S[16 i + 4 q + r][c0 + 16 j + n] in sacc[i][j][r]; requested after the
    // chunk's inputs, so the state streams in while the S-independent part
    // of the chunk is computed
    f32x4 sacc[NIB][NTJ];
    const float *S0 = P.S0 ? P.S0 + (long)bh * DK * DV : nullptr;
#pragma unroll
    for (int i = 0; i < NIB; ++i)
#pragma unroll
        for (int j = 0; j < NTJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[i][j][r] = S0 ? S0[(long)(16 * i + 4 * q + r) * DV + c0 + 16 * j + n] : 0.f;
    float p_reg = 0.f;               // variance of channel tid (KDN), of the head (ISO)
    if (KDN && tid < DK)
        p_reg = P.p0[(long)bh * DK + tid];
    if (ISO && tid == 0)
        p_reg = P.p0[bh];

    {
        // ---- 1. the chunk's raw tiles into LDS
        {
            if (st_t < TC) {
                *reinterpret_cast<uint4 *>(Kr + st_t * PK + st_c) = rk;
                *reinterpret_cast<uint4 *>(Qr + st_t * PK + st_c) = rq;
                if (VDECAY)
                    *reinterpret_cast<uint4 *>(Ar + st_t * PK + st_c) = ra;
                if (KDN || ISO)
                    *reinterpret_cast<uint4 *>(Xr + st_t * PK + st_c) = rx;
            }
            if (tid < TC) {
                s_r[tid] = rr;
                s_b[tid] = rb;
                s_a[tid] = rga;
            }
            if (tid == 0)
                *s_flag = 0;
        }
        __syncthreads();

        // ---- 2. write strengths
        if constexpr (KDN) {
            // variance chain per key channel (page "给记忆装一个信任度探测器 ...",
            // section "对角近似：把矩阵压扁成一个向量"):
            //   p- = a^2 p + xi,  u = p- k,  p = p- r / (r + mu p- k^2)
            if (tid < DK) {
                const int i = tid;
                float pc = p_reg;
#pragma unroll
                for (int t = 0; t < TC; ++t) {
                    const float k = to_f32(Kr[t * PK + i]), a = to_f32(Ar[t * PK + i]);
                    const float x = to_f32(Xr[t * PK + i]), r = s_r[t];
                    const float pm = fmaf(a * a, pc, x);
                    U32[t * PU + i] = pm * k;
                    const float den = fmaf(P.mu * k * k, pm, r);
                    pc = (den != 0.f) ? pm * r * fast_rcp(den) : pm;
                }
                p_reg = pc;
            }
            __syncthreads();
            // innovation variances s_t = r_t + sum_i u_ti k_ti (16 threads per token)
            {
                constexpr int CPT = DK / 16;
                const int t = tid >> 4, part = tid & 15;
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    const int i = part * CPT + c;
                    acc += U32[t * PU + i] * to_f32(Kr[t * PK + i]);
                }
                acc = row16_sum_last(acc);
                if (part == 15) {
                    const float s = s_r[t] + acc;
                    s_invs[t] = (s != 0.f) ? 1.f / s : 0.f;
                }
            }
        } else if constexpr (ISO) {
            // per-token channel sums, then the head variance token by token
            // (section "各向同性近似：把整个头压缩成一个数"):
            //   p- = mean(a^2) p + mean(xi),  beta = p- / (r + p- |k|^2),
            //   p = p- r / (r + (mu / d_k) p- |k|^2)
            {
                constexpr int CPT = DK / 16;
                const int t = tid >> 4, part = tid & 15;
                float sa = 0.f, sx = 0.f, sk = 0.f;
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    const int i = part * CPT + c;
                    const float a = to_f32(Ar[t * PK + i]), k = to_f32(Kr[t * PK + i]);
                    sa = fmaf(a, a, sa);
                    sx += to_f32(Xr[t * PK + i]);
                    sk = fmaf(k, k, sk);
                }
                sa = row16_sum_last(sa);
                sx = row16_sum_last(sx);
                sk = row16_sum_last(sk);
                if (part == 15) {
                    s_ia2[t] = sa * (1.f / DK);
                    s_ixm[t] = sx * (1.f / DK);
                    s_ikk[t] = sk;
                }
            }
            __syncthreads();
            if (tid == 0) {
                float pc = p_reg;
                for (int t = 0; t < TC; ++t) {
                    const float kk = s_ikk[t], r = s_r[t];
                    const float pm = fmaf(s_ia2[t], pc, s_ixm[t]);
                    const float sv = fmaf(pm, kk, r);
                    s_b[t] = (t < L && sv != 0.f) ? pm / sv : 0.f;
                    const float den = fmaf(P.mu * (1.f / DK) * pm, kk, r);
                    pc = (den != 0.f) ? pm * r / den : pm;
                }
                p_reg = pc;
            }
        }
        __syncthreads();

        // ---- 3. decays and scaled operands, one thread per key channel:
        //   gamma_t = prod_{r<=t} a_r,  K~ = gamma k,  Q~ = gamma q,
        //   W' = w / gamma,  W~^T[i][t] = (prod_{r>t} a_r) w_t
        if (tid < DK) {
            const int i = tid;
            const int g = i >> 5, wi = i & 31;
            const int qq = (wi & 15) >> 2;           // k-slot of the permuted order
            const int ee = (wi & 3) + (wi & 16 ? 4 : 0);
            auto wval = [&](int t) {
                const float k = to_f32(Kr[t * PK + i]);
                if constexpr (KDN)
                    return U32[t * PU + i] * s_invs[t];
                else
                    return s_b[t] * k;
            };
            auto aval = [&](int t) {
                if constexpr (VDECAY)
                    return to_f32(Ar[t * PK + i]);
                else if constexpr (VAR == GATED_DELTANET)
                    return s_a[t];
                else
                    return 1.f;
            };
            float gam = 1.f;
            bool low = false;
#pragma unroll
            for (int t = 0; t < TC; ++t) {
                gam *= aval(t);
                low |= !(gam >= SHORT_DECAY_FLOOR);
                const float w = wval(t);
                const int f = ((g * 64 + qq * 16 + t) * 8 + ee);   // fragment element
                KF[f] = static_cast<bf16>(gam * to_f32(Kr[t * PK + i]));
                QF[f] = static_cast<bf16>(gam * to_f32(Qr[t * PK + i]));
                WF[f] = static_cast<bf16>(DECAY ? w * fast_rcp(gam) : w);
            }
            sgc[i] = gam;
            float suf = 1.f;
#pragma unroll
            for (int t = TC - 1; t >= 0; --t) {
                // A operand of the K = 16 S update: row i, k-slot t
                WT[((i >> 4) * 64 + (t >> 2) * 16 + (i & 15)) * 4 + (t & 3)] =
                    static_cast<bf16>(suf * wval(t));
                suf *= aval(t);
            }
            if (DECAY && low)
                *s_flag = 1;
        }
        __syncthreads();

        // ---- 4. A_kk (strictly lower) and A_qk (lower with the diagonal)
        const bool exact = DECAY && *s_flag != 0;
        if (!exact) {
            if (wv < 2) {
                const bf16x8 *X = reinterpret_cast<const bf16x8 *>(wv == 0 ? KF : QF);
                const bf16x8 *W = reinterpret_cast<const bf16x8 *>(WF);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < GK; ++g)
                    acc = mfma32(X[g * 64 + lane], W[g * 64 + lane], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * q + r, s = n;
                    if (wv == 0)
                        Akk[t * TC + s] = s < t ? acc[r] : 0.f;
                    else
                        AQ[((s >> 2) * 16 + t) * 4 + (s & 3)] =
                            static_cast<bf16>(s <= t ? acc[r] : 0.f);
                }
            }
        } else {
            // some channel decays below the floor inside the chunk: the decay
            // ratios are multiplied out directly (no 1/gamma)
            const int t = tid >> 4, s = tid & 15;
            float akk = 0.f, aqk = 0.f;
            if (s <= t) {
                for (int i = 0; i < DK; ++i) {
                    float R = 1.f;
                    for (int r = s + 1; r <= t; ++r)
                        R *= VDECAY ? to_f32(Ar[r * PK + i]) : s_a[r];
                    const float k_s = to_f32(Kr[s * PK + i]);
                    const float w = KDN ? U32[s * PU + i] * s_invs[s] : s_b[s] * k_s;
                    akk += to_f32(Kr[t * PK + i]) * w * R;
                    aqk += to_f32(Qr[t * PK + i]) * w * R;
                }
            }
            Akk[t * TC + s] = s < t ? akk : 0.f;
            AQ[((s >> 2) * 16 + t) * 4 + (s & 3)] = static_cast<bf16>(s <= t ? aqk : 0.f);
        }
        __syncthreads();

        // ---- 5. T = (I + A_kk)^-1 by forward substitution, one column per
        //      lane of wave 0 (fp32), then T as the A operand of K = 16
        if (wv == 0 && lane < TC) {
            const int s = lane;
            float tc[TC];
#pragma unroll
            for (int t = 0; t < TC; ++t) {
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < t; ++k)
                    acc = fmaf(Akk[t * TC + k], tc[k], acc);
                tc[t] = t < s ? 0.f : (t == s ? 1.f : -acc);
            }
#pragma unroll
            for (int t = 0; t < TC; ++t)
                TF[((s >> 2) * 16 + t) * 4 + (s & 3)] = static_cast<bf16>(tc[t]);
        }
        __syncthreads();

        // ---- 6. this wave's columns: U, E, O and the S update
        {
            const bf16x8 *KFv = reinterpret_cast<const bf16x8 *>(KF);
            const bf16x8 *QFv = reinterpret_cast<const bf16x8 *>(QF);
            const s16x4 tf = reinterpret_cast<const s16x4 *>(TF)[lane];
            const s16x4 af = reinterpret_cast<const s16x4 *>(AQ)[lane];
            bf16x8 sb[GK][NTJ];
#pragma unroll
            for (int g = 0; g < GK; ++g)
#pragma unroll
                for (int j = 0; j < NTJ; ++j)
                    sb[g][j] = pack8(sacc[2 * g][j], sacc[2 * g + 1][j]);
            f32x4 ua[NTJ], oa[NTJ];
#pragma unroll
            for (int j = 0; j < NTJ; ++j) {
                ua[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                oa[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int g = 0; g < GK; ++g) {
                const bf16x8 kf = KFv[g * 64 + lane], qf = QFv[g * 64 + lane];
#pragma unroll
                for (int j = 0; j < NTJ; ++j) {
                    ua[j] = mfma32(kf, sb[g][j], ua[j]);
                    oa[j] = mfma32(qf, sb[g][j], oa[j]);
                }
            }
            s16x4 eb[NTJ];
#pragma unroll
            for (int j = 0; j < NTJ; ++j) {
                // U = V - K~ S (rows past the sequence end read as 0)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ua[j][r] = rv[j][r] - ua[j][r];
                // E = T U
                const f32x4 ea = mfma16(tf, pack4(ua[j]), f32x4{0.f, 0.f, 0.f, 0.f});
                eb[j] = pack4(ea);
                // O = Q~ S + A_qk E
                oa[j] = mfma16(af, eb[j], oa[j]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * q + r;
                    if (t < L)
                        go[seqv + (long)t * hdv + c0 + 16 * j + n] =
                            static_cast<bf16>(oa[j][r]);
                }
            }
            // S <- diag(gamma) S + W~^T E
            const s16x4 *WTv = reinterpret_cast<const s16x4 *>(WT);
#pragma unroll
            for (int i = 0; i < NIB; ++i) {
                const s16x4 wt = WTv[i * 64 + lane];
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(sgc + 16 * i + 4 * q);
#pragma unroll
                for (int j = 0; j < NTJ; ++j) {
                    if (DECAY) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            sacc[i][j][r] *= gm[r];
                    }
                    sacc[i][j] = mfma16(wt, eb[j], sacc[i][j]);
                }
            }
        }
    }

    float *So = P.S_out + (long)bh * DK * DV;
#pragma unroll
    for (int i = 0; i < NIB; ++i)
#pragma unroll
        for (int j = 0; j < NTJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                So[(long)(16 * i + 4 * q + r) * DV + c0 + 16 * j + n] = sacc[i][j][r];
    if (KDN && tid < DK)
        P.p_out[(long)bh * DK + tid] = p_reg;
    if (ISO && tid == 0)
        P.p_out[bh] = p_reg;
}

template <int VAR, int DK, int DV>
static hipError_t launch_short_one(const PrefillParams &P, hipStream_t st) {
    const dim3 grid((unsigned)((long)P.B * P.H)), block(NT);
    hipLaunchKernelGGL((prefill_short_kernel<VAR, DK, DV>), grid, block, 0, st, P);
    return hipGetLastError();
}

template <int VAR>
static hipError_t launch_short_v(const PrefillParams &P, hipStream_t st) {
    if (P.dk == 128 && P.dv == 128) return launch_short_one<VAR, 128, 128>(P, st);
    if (P.dk == 128 && P.dv == 64) return launch_short_one<VAR, 128, 64>(P, st);
    if (P.dk == 64 && P.dv == 128) return launch_short_one<VAR, 64, 128>(P, st);
    if (P.dk == 64 && P.dv == 64) return launch_short_one<VAR, 64, 64>(P, st);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_short(const PrefillParams &P, hipStream_t st) {
    if (!P.bf16)
        return hipErrorInvalidValue;
    switch (P.variant) {
    case DELTANET: return launch_short_v<DELTANET>(P, st);
    case GATED_DELTANET: return launch_short_v<GATED_DELTANET>(P, st);
    case KDA: return launch_short_v<KDA>(P, st);
    case DIAG_KDN: return launch_short_v<DIAG_KDN>(P, st);
    case ISO_KDN: return launch_short_v<ISO_KDN>(P, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace kdn
