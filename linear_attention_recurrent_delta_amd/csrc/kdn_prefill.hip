// kdn_prefill.hip -- chunkwise prefill of the delta-rule family (gfx950).
//
// Chunk algebra (derived from the token recurrence; the chunked form is exact,
// page "معماری KDA: حذف تداخل حافظه با قانون دلتا در توالی‌های بلند", section
// "حل مشکل وابستگی علی": provisional errors, then a causal triangular solve,
// with interaction matrices A_kk and A_qk that carry the cumulative decay).
// For a chunk of C tokens entering with state S0, per key channel i:
//   gamma_t = prod_{r<=t} a_r,   K~ = gamma (.) K,   Q~ = gamma (.) Q,
//   A_kk[t,s] = sum_i k_ti w_si gamma_ti / gamma_si          (s <  t)
//   A_qk[t,s] = sum_i q_ti w_si gamma_ti / gamma_si          (s <= t)
//   E  = (I + A_kk)^-1 (V - K~ S0)             errors, causally resolved
//   O  = Q~ S0 + A_qk E                         outputs o_t = S_t^T q_t
//   S  = diag(gamma_C) S0 + W~^T E,  W~_s = (gamma_C / gamma_s) (.) w_s.
// Write vectors: w = beta k (DeltaNet, Gated DeltaNet, KDA) or the diagonal
// Kalman gain (page "给记忆装一个信任度探测器：Kalman Delta Networks 如何让AI知道自己
// "记得准不准"", section "对角近似：把矩阵压扁成一个向量"), whose variance recursion
// does not depend on S and runs per channel inside the chunk.
//
// Work split: one workgroup (4 waves) owns one (batch, head, d_v block of NV
// columns) and walks all chunks in order; the d_k x NV slice of S stays in
// MFMA accumulator registers in float32 for the whole sequence.  Sibling
// workgroups of a head (different d_v blocks) repeat the S-independent work
// (decay prep, gains, A matrices, triangular inverse) so that the grid fills
// the 256 CUs; they are placed on one XCD so that q/k/gate reads hit its L2.
//
// Per chunk:
//   1  stage raw q, k, alpha, xi tiles and the v block in LDS (16 B loads);
//   2  column pass, one thread per key channel: cumulative decay, scaled
//      operands K~, Q~, W' = w / gamma and W~ (transposed), KDN gains;
//   3  A_kk, A_qk on MFMA from K~ W'^T and Q~ W'^T (exact elementwise
//      fallback when a channel decays below 2^-90 inside the chunk);
//   4  T = (I + A_kk)^-1: 16x16 diagonal blocks by forward substitution, then
//      the off-diagonal blocks level by level;
//   5  U = V - K~ S on MFMA;   6  E = T U on MFMA;
//   7  O = Q~ S + A_qk E (stored), S = gamma_C S + W~^T E on MFMA;
//   8  S rounded to the operand type for the next chunk's products.
#include "kdn_device.h"
#include "kdn_launch.h"

namespace kdn {

#ifdef KDN_PREFILL_VARIANT
// Below this cumulative in-chunk decay the 1/gamma operand scaling is not
// used (it would leave the float range); the chunk takes the exact path.
#define KDN_DECAY_FLOOR 8.077935669463161e-28f   /* 2^-90 */

template <typename E, int VAR, int DK, int NV, int C>
struct PrefillLayout {
    static constexpr int NT = 256;
    static constexpr int PADE = 16 / (int)sizeof(E);
    static constexpr int PK = DK + PADE;     // pitch of [*][DK] operands
    static constexpr int PC = C + PADE;      // pitch of [*][C] operands
    static constexpr int PV = NV + PADE;     // pitch of the staged v block
    static constexpr int PA = C + 4;         // pitch of the fp32 A_kk
    static constexpr int PP = DK + 4;        // pitch of the fp32 KDN scratch
    static constexpr int NB = C / 16;        // 16-row blocks per chunk
    static constexpr bool DECAY = VAR != DELTANET;
    static constexpr bool VDECAY = VAR == KDA || VAR == DIAG_KDN;
    static constexpr bool KDN = VAR == DIAG_KDN;

    static constexpr int SZ_CK = C * PK * (int)sizeof(E);
    static constexpr int OFF_KT = 0;
    static constexpr int OFF_QT = OFF_KT + SZ_CK;
    static constexpr int OFF_WP = OFF_QT + SZ_CK;
    static constexpr int OFF_ALP = OFF_WP + SZ_CK;
    static constexpr int OFF_WTT = OFF_ALP + (VDECAY ? SZ_CK : 0);
    static constexpr int SZ_WTT = DK * PC * (int)sizeof(E);
    static constexpr int OFF_ST = OFF_WTT + SZ_WTT;
    static constexpr int OFF_VR = OFF_ST + NV * PK * (int)sizeof(E);
    // A_kk, T, A_qk, U^T, E^T are contiguous: the KDN scratch aliases them.
    static constexpr int OFF_AKK = OFF_VR + C * PV * (int)sizeof(E);
    static constexpr int OFF_TM = OFF_AKK + C * PA * 4;
    static constexpr int OFF_AQ = OFF_TM + C * PC * (int)sizeof(E);
    static constexpr int OFF_UT = OFF_AQ + C * PC * (int)sizeof(E);
    static constexpr int OFF_ET = OFF_UT + NV * PC * (int)sizeof(E);
    static constexpr int END_ET = OFF_ET + NV * PC * (int)sizeof(E);
    static constexpr int END_PK2 = OFF_AKK + (KDN ? C * PP * 4 : 0);
    static constexpr int OFF_SM = END_ET > END_PK2 ? END_ET : END_PK2;
    // small fp32 vectors
    static constexpr int SM_BETA = 0, SM_R = C, SM_ALPH = 2 * C, SM_INVS = 3 * C,
                         SM_GC = 4 * C, SM_FLAG = 4 * C + DK;
    static constexpr int SZ_SM = (4 * C + DK + 4) * 4;
    static constexpr int TOTAL = OFF_SM + SZ_SM;

    static_assert(TOTAL <= 163840, "prefill LDS budget");
    static_assert(!KDN || C * PP * 4 <= OFF_SM - OFF_AKK, "KDN scratch alias");
    static_assert(!KDN || C * PK <= DK * PC, "xi staging alias");
    static_assert((NB - 1) * 256 * 4 <= SZ_CK, "level scratch (aliases W')");
    static_assert(C % 16 == 0 && NV % 16 == 0 && DK % 16 == 0, "tiles");
    static_assert(NT % C == 0, "row reduction layout");
};

// Copy ROWS x D elements (rows t < L from global, stride `stride` elements)
// into LDS rows of pitch `pitch`; rows t >= L are filled with `pad`.
template <typename T, int D, int ROWS>
__device__ __forceinline__ void stage_rows(T *dst, int pitch, const T *src,
                                           long stride, int L, float pad,
                                           int tid) {
    constexpr int VN = 16 / (int)sizeof(T);
    constexpr int VPR = D / VN;
    static_assert(VPR * VN == D, "row width");
    const T pv = from_f32<T>(pad);
    for (int x = tid; x < ROWS * VPR; x += 256) {
        const int t = x / VPR, c = x % VPR;
        uint4 raw;
        if (t < L) {
            raw = *reinterpret_cast<const uint4 *>(src + (long)t * stride + c * VN);
        } else {
            T tmp[VN];
#pragma unroll
            for (int e = 0; e < VN; ++e)
                tmp[e] = pv;
            raw = *reinterpret_cast<const uint4 *>(tmp);
        }
        *reinterpret_cast<uint4 *>(dst + t * pitch + c * VN) = raw;
    }
}

template <typename E>
__device__ __forceinline__ float ld(const E *p) { return to_f32(*p); }

template <typename E, int VAR, int DK, int NV, int C>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams P) {
    using LY = PrefillLayout<E, VAR, DK, NV, C>;
    constexpr int PK = LY::PK, PC = LY::PC, PV = LY::PV, PA = LY::PA,
                  PP = LY::PP, NB = LY::NB;
    constexpr bool DECAY = LY::DECAY, VDECAY = LY::VDECAY, KDN = LY::KDN;
    constexpr int NTJ = NV / 16;                // value tiles
    constexpr int NTI = DK / 16;                // key tiles
    constexpr int NS = NTI * NTJ / 4;           // S tiles per wave
    static_assert(NS * 4 == NTI * NTJ, "S tiles per wave");
    constexpr int KS = Mma<E>::KSTEP;

    __shared__ __attribute__((aligned(16))) char smem[LY::TOTAL];
    E *Kt = reinterpret_cast<E *>(smem + LY::OFF_KT);
    E *Qt = reinterpret_cast<E *>(smem + LY::OFF_QT);
    E *Wp = reinterpret_cast<E *>(smem + LY::OFF_WP);
    E *ALP = reinterpret_cast<E *>(smem + LY::OFF_ALP);
    E *WtT = reinterpret_cast<E *>(smem + LY::OFF_WTT);
    E *XR = WtT;                                   // KDN: raw xi staging
    E *ST = reinterpret_cast<E *>(smem + LY::OFF_ST);
    E *VR = reinterpret_cast<E *>(smem + LY::OFF_VR);
    float *Akk = reinterpret_cast<float *>(smem + LY::OFF_AKK);
    float *PK2 = Akk;                              // KDN: p- k^2 scratch
    E *Tm = reinterpret_cast<E *>(smem + LY::OFF_TM);
    E *AQ = reinterpret_cast<E *>(smem + LY::OFF_AQ);
    E *UT = reinterpret_cast<E *>(smem + LY::OFF_UT);
    E *ET = reinterpret_cast<E *>(smem + LY::OFF_ET);
    float *Pl = reinterpret_cast<float *>(smem + LY::OFF_WP);  // level scratch
    float *sm = reinterpret_cast<float *>(smem + LY::OFF_SM);
    float *s_beta = sm + LY::SM_BETA, *s_r = sm + LY::SM_R,
          *s_alph = sm + LY::SM_ALPH, *s_invs = sm + LY::SM_INVS,
          *s_gc = sm + LY::SM_GC;
    int *s_flag = reinterpret_cast<int *>(sm + LY::SM_FLAG);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;

    // Workgroup -> (batch*head, value block).  Dispatch is round-robin over
    // the 8 XCDs; place the value blocks of one head on one XCD.
    const int nvb = P.dv / NV;
    const int G = gridDim.x;
    int lid = blockIdx.x;
    if ((G & 7) == 0 && ((G >> 3) % nvb) == 0)
        lid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int bh = lid / nvb, vb = lid % nvb;
    const int b = bh / P.H, h = bh % P.H;
    const int v0 = vb * NV;
    const int T = P.T, H = P.H, DV = P.dv;

    const E *gq = static_cast<const E *>(P.q);
    const E *gk = static_cast<const E *>(P.k);
    const E *gv = static_cast<const E *>(P.v);
    const E *ga = static_cast<const E *>(P.alpha);
    const E *gb = static_cast<const E *>(P.beta);
    const E *gx = static_cast<const E *>(P.xi);
    const E *gr = static_cast<const E *>(P.r);

    // ---- S slice in accumulator layout: tile u of this wave is
    //      (ti, tj) = divmod(wv + 4u, NTJ); acc[r] = S[ti*16 + (lane>>4)*4 + r]
    //                                                 [tj*16 + (lane&15)].
    f32x4 sacc[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int tau = wv + 4 * u, ti = tau / NTJ, tj = tau % NTJ;
        const int j = tj * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ti * 16 + (lane >> 4) * 4 + r;
            sacc[u][r] = P.S0 ? P.S0[((long)bh * DK + i) * DV + v0 + j] : 0.f;
            ST[j * PK + i] = from_f32<E>(sacc[u][r]);
        }
    }
    float p_reg = 0.f;                 // KDN variance of channel tid
    if (KDN && tid < DK)
        p_reg = P.p0[(long)bh * DK + tid];

    const long sk_ = (long)H * DK;     // token stride of q/k/alpha/xi
    const long sv_ = (long)H * DV;     // token stride of v/o

    for (int c0 = 0; c0 < T; c0 += C) {
        const int L = min(C, T - c0);
        const long tok0 = ((long)b * T + c0) * H + h;   // (b, c0, h)

        // ---------------- 1. stage raw tiles ----------------
        stage_rows<E, DK, C>(Kt, PK, gk + tok0 * DK, sk_, L, 0.f, tid);
        stage_rows<E, DK, C>(Qt, PK, gq + tok0 * DK, sk_, L, 0.f, tid);
        if (VDECAY)
            stage_rows<E, DK, C>(ALP, PK, ga + tok0 * DK, sk_, L, 1.f, tid);
        if (KDN)
            stage_rows<E, DK, C>(XR, PK, gx + tok0 * DK, sk_, L, 0.f, tid);
        stage_rows<E, NV, C>(VR, PV, gv + tok0 * DV + v0, sv_, L, 0.f, tid);
        if (tid < C) {
            const int t = tid;
            const long ti = tok0 + (long)t * H;
            if (!KDN)
                s_beta[t] = t < L ? ld(gb + ti) : 0.f;
            else
                s_r[t] = t < L ? ld(gr + ti) : 1.f;
            if (VAR == GATED_DELTANET)
                s_alph[t] = t < L ? ld(ga + ti) : 1.f;
        }
        if (tid == 0)
            *s_flag = 0;
        __syncthreads();

        // ---------------- 2. column pass ----------------
        float wreg[C];
        if (tid < DK) {
            const int i = tid;
            float g = 1.f;
#pragma unroll
            for (int t = 0; t < C; ++t) {
                const float kk = ld(Kt + t * PK + i);
                const float qq = ld(Qt + t * PK + i);
                float a = 1.f;
                if (VAR == GATED_DELTANET) a = s_alph[t];
                if (VDECAY) a = ld(ALP + t * PK + i);
                if (DECAY) {
                    g *= a;
                    Kt[t * PK + i] = from_f32<E>(g * kk);
                    Qt[t * PK + i] = from_f32<E>(g * qq);
                }
                if (KDN) {
                    if (t < L) {
                        const float pm = a * a * p_reg + ld(XR + t * PK + i);
                        const float r = s_r[t];
                        const float u = pm * kk;
                        PK2[t * PP + i] = u * kk;
                        const float den = r + P.mu * pm * kk * kk;
                        p_reg = (den != 0.f) ? pm * r / den : pm;
                        wreg[t] = u;
                    } else {
                        PK2[t * PP + i] = 0.f;
                        wreg[t] = 0.f;
                    }
                } else {
                    wreg[t] = s_beta[t] * kk;
                }
            }
            if (DECAY && !(g >= KDN_DECAY_FLOOR))
                *s_flag = 1;
        }
        __syncthreads();
        if (KDN) {
            // innovation variances s_t = r_t + sum_i p-_ti k_ti^2
            constexpr int TPR = 256 / C;          // threads per token row
            constexpr int CPT = DK / TPR;          // channels per thread
            const int t = tid / TPR, part = tid % TPR;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CPT; ++c)
                acc += PK2[t * PP + part * CPT + c];
#pragma unroll
            for (int off = TPR / 2; off >= 1; off >>= 1)
                acc += __shfl_xor(acc, off, WAVE);
            if (part == 0) {
                const float s = s_r[t] + acc;
                s_invs[t] = (s != 0.f) ? 1.f / s : 0.f;
            }
            __syncthreads();
            if (tid < DK) {
#pragma unroll
                for (int t2 = 0; t2 < C; ++t2)
                    wreg[t2] *= s_invs[t2];
            }
        }
        const bool fb = DECAY && (*s_flag != 0);
        if (tid < DK) {
            const int i = tid;
            float g = 1.f;
#pragma unroll
            for (int t = 0; t < C; ++t) {
                float a = 1.f;
                if (VAR == GATED_DELTANET) a = s_alph[t];
                if (VDECAY) a = ld(ALP + t * PK + i);
                g *= a;
                Wp[t * PK + i] = from_f32<E>((DECAY && !fb) ? wreg[t] / g : wreg[t]);
            }
            s_gc[i] = g;
            float sg = 1.f;
#pragma unroll
            for (int t = C - 1; t >= 0; --t) {
                WtT[i * PC + t] = from_f32<E>(sg * wreg[t]);
                float a = 1.f;
                if (VAR == GATED_DELTANET) a = s_alph[t];
                if (VDECAY) a = ld(ALP + t * PK + i);
                sg *= a;
            }
        }
        __syncthreads();

        // ---------------- 3. interaction matrices ----------------
        constexpr int NL = NB * (NB + 1) / 2;
        if (!fb) {
            for (int x = wv; x < 2 * NL; x += 4) {
                const int which = x >= NL;
                int idx = x - which * NL, mi = 0;
                while (idx > mi) { idx -= mi + 1; ++mi; }
                const int ni = idx;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                mma_tile<E>(acc, (which ? Qt : Kt) + mi * 16 * PK, PK,
                            Wp + ni * 16 * PK, PK, DK, lane);
                const int s = ni * 16 + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = mi * 16 + (lane >> 4) * 4 + r;
                    if (which)
                        AQ[t * PC + s] = from_f32<E>(s <= t ? acc[r] : 0.f);
                    else
                        Akk[t * PA + s] = s < t ? acc[r] : 0.f;
                }
            }
        } else if constexpr (DECAY) {
            // Exact path: reload raw k, q; products of the decays directly.
            stage_rows<E, DK, C>(Kt, PK, gk + tok0 * DK, sk_, L, 0.f, tid);
            stage_rows<E, DK, C>(Qt, PK, gq + tok0 * DK, sk_, L, 0.f, tid);
            __syncthreads();
            for (int pidx = tid; pidx < C * C; pidx += 256) {
                const int t = pidx / C, s = pidx % C;
                float akk = 0.f, aqk = 0.f;
                if (s <= t) {
                    for (int i = 0; i < DK; ++i) {
                        float R = 1.f;
                        for (int rr = s + 1; rr <= t; ++rr)
                            R *= (VAR == GATED_DELTANET) ? s_alph[rr]
                                                         : ld(ALP + rr * PK + i);
                        const float ws = ld(Wp + s * PK + i) * R;
                        akk += ld(Kt + t * PK + i) * ws;
                        aqk += ld(Qt + t * PK + i) * ws;
                    }
                }
                Akk[t * PA + s] = s < t ? akk : 0.f;
                AQ[t * PC + s] = from_f32<E>(s <= t ? aqk : 0.f);
            }
            __syncthreads();
            if (tid < DK) {       // back to the decay-scaled operands
                const int i = tid;
                float g = 1.f;
                for (int t = 0; t < C; ++t) {
                    float a = (VAR == GATED_DELTANET) ? s_alph[t]
                                                      : ld(ALP + t * PK + i);
                    g *= a;
                    Kt[t * PK + i] = from_f32<E>(g * ld(Kt + t * PK + i));
                    Qt[t * PK + i] = from_f32<E>(g * ld(Qt + t * PK + i));
                }
            }
        }
        // zero the blocks above the diagonal of A_qk and T (MFMA K ranges
        // may cover them)
        for (int x = tid; x < C * C; x += 256) {
            const int t = x / C, s = x % C;
            if ((s >> 4) > (t >> 4)) {
                AQ[t * PC + s] = from_f32<E>(0.f);
                Tm[t * PC + s] = from_f32<E>(0.f);
            }
        }
        __syncthreads();

        // ---------------- 5. U = V - K~ S  (overlaps 4a) ----------------
        constexpr int NTU = NB * NTJ;
        for (int x = wv; x < NTU; x += 4) {
            const int mi = x / NTJ, nj = x % NTJ;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile<E>(acc, Kt + mi * 16 * PK, PK, ST + nj * 16 * PK, PK, DK, lane);
            const int j = nj * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = mi * 16 + (lane >> 4) * 4 + r;
                UT[j * PC + t] = from_f32<E>(ld(VR + t * PV + j) - acc[r]);
            }
        }
        // ---------------- 4a. diagonal blocks of T ----------------
        if (wv == 0 && (lane >> 4) < NB) {
            const int blk = lane >> 4, j = lane & 15, o0 = blk * 16;
            float xv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m)
                    acc += Akk[(o0 + r) * PA + o0 + m] * xv[m];
                xv[r] = (r == j) ? 1.f : ((r < j) ? 0.f : -acc);
                Tm[(o0 + r) * PC + o0 + j] = from_f32<E>(xv[r]);
            }
        }
        __syncthreads();
        // ---------------- 4b. off-diagonal blocks of T ----------------
        // T[I,J] = -T[I,I] * sum_{K=J}^{I-1} A[I,K] T[K,J], level d = I - J.
        for (int d = 1; d < NB; ++d) {
            const int nbl = NB - d;
            for (int e = tid; e < nbl * 256; e += 256) {
                const int I = d + e / 256, rr = (e % 256) / 16, cc = e % 16;
                const int J = I - d;
                float acc = 0.f;
                for (int Kb = J; Kb < I; ++Kb)
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        acc += Akk[(I * 16 + rr) * PA + Kb * 16 + m] *
                               ld(Tm + (Kb * 16 + m) * PC + J * 16 + cc);
                Pl[e] = acc;
            }
            __syncthreads();
            for (int e = tid; e < nbl * 256; e += 256) {
                const int I = d + e / 256, rr = (e % 256) / 16, cc = e % 16;
                const int J = I - d;
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    acc += ld(Tm + (I * 16 + rr) * PC + I * 16 + m) *
                           Pl[(e / 256) * 256 + m * 16 + cc];
                Tm[(I * 16 + rr) * PC + J * 16 + cc] = from_f32<E>(-acc);
            }
            __syncthreads();
        }
        // ---------------- 6. E = T U ----------------
        for (int x = wv; x < NTU; x += 4) {
            const int mi = x / NTJ, nj = x % NTJ;
            const int kc = min(C, ((mi + 1) * 16 + KS - 1) / KS * KS);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile<E>(acc, Tm + mi * 16 * PC, PC, UT + nj * 16 * PC, PC, kc, lane);
            const int j = nj * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = mi * 16 + (lane >> 4) * 4 + r;
                ET[j * PC + t] = from_f32<E>(acc[r]);
            }
        }
        __syncthreads();

        // ---------------- 7. outputs and state ----------------
        E *go = static_cast<E *>(P.o);
        for (int x = wv; x < NTU; x += 4) {
            const int mi = x / NTJ, nj = x % NTJ;
            const int kc = min(C, ((mi + 1) * 16 + KS - 1) / KS * KS);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile<E>(acc, Qt + mi * 16 * PK, PK, ST + nj * 16 * PK, PK, DK, lane);
            mma_tile<E>(acc, AQ + mi * 16 * PC, PC, ET + nj * 16 * PC, PC, kc, lane);
            const int j = nj * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = mi * 16 + (lane >> 4) * 4 + r;
                if (t < L)
                    go[(tok0 + (long)t * H) * DV + v0 + j] = from_f32<E>(acc[r]);
            }
        }
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int tau = wv + 4 * u, ti = tau / NTJ, tj = tau % NTJ;
            if (DECAY) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sacc[u][r] *= s_gc[ti * 16 + (lane >> 4) * 4 + r];
            }
            mma_tile<E>(sacc[u], WtT + ti * 16 * PC, PC, ET + tj * 16 * PC, PC, C, lane);
        }
        __syncthreads();

        // ---------------- 8. S for the next chunk's products ----------------
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int tau = wv + 4 * u, ti = tau / NTJ, tj = tau % NTJ;
            const int j = tj * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ST[j * PK + ti * 16 + (lane >> 4) * 4 + r] = from_f32<E>(sacc[u][r]);
        }
    }

    // ---- final state
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int tau = wv + 4 * u, ti = tau / NTJ, tj = tau % NTJ;
        const int j = tj * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ti * 16 + (lane >> 4) * 4 + r;
            P.S_out[((long)bh * DK + i) * DV + v0 + j] = sacc[u][r];
        }
    }
    if (KDN && vb == 0 && tid < DK)
        P.p_out[(long)bh * DK + tid] = p_reg;
}

#endif  // KDN_PREFILL_VARIANT

// ---------------------------------------------------------------------------
// Host-side dispatch.  This file is compiled once per variant
// (KDN_PREFILL_VARIANT = 0..3, each unit instantiates that variant's kernels)
// and once with KDN_PREFILL_DISPATCH for the entry point below.
// ---------------------------------------------------------------------------
#ifdef KDN_PREFILL_VARIANT
template <typename E, int VAR, int DK, int NV, int C>
static hipError_t launch_one(const PrefillParams &P, hipStream_t st) {
    const long heads = (long)P.B * P.H;
    const dim3 grid((unsigned)(heads * (P.dv / NV))), block(256);
    hipLaunchKernelGGL((prefill_kernel<E, VAR, DK, NV, C>), grid, block, 0, st, P);
    return hipGetLastError();
}

template <typename E, int VAR, int DK, int C>
static hipError_t launch_nv(const PrefillParams &P, hipStream_t st, int nv) {
    if (nv == 16)
        return launch_one<E, VAR, DK, 16, C>(P, st);
    if constexpr (sizeof(E) == 2) {
        if (nv == 32)
            return launch_one<E, VAR, DK, 32, C>(P, st);
    }
    return hipErrorInvalidValue;
}

template <typename E, int VAR>
static hipError_t launch_var(const PrefillParams &P, hipStream_t st, int nv) {
    if (P.dk == 128 && P.chunk == 64) {
        if constexpr (sizeof(E) == 2)
            return launch_nv<E, VAR, 128, 64>(P, st, nv);
        return hipErrorInvalidValue;
    }
    if (P.dk == 128 && P.chunk == 32) return launch_nv<E, VAR, 128, 32>(P, st, nv);
    if (P.dk == 64 && P.chunk == 64) return launch_nv<E, VAR, 64, 64>(P, st, nv);
    if (P.dk == 64 && P.chunk == 32) return launch_nv<E, VAR, 64, 32>(P, st, nv);
    return hipErrorInvalidValue;
}

#define KDN_CAT2(a, b) a##b
#define KDN_CAT(a, b) KDN_CAT2(a, b)
hipError_t KDN_CAT(launch_prefill_v, KDN_PREFILL_VARIANT)(const PrefillParams &P,
                                                          hipStream_t st, int nv) {
    return P.bf16 ? launch_var<bf16, KDN_PREFILL_VARIANT>(P, st, nv)
                  : launch_var<float, KDN_PREFILL_VARIANT>(P, st, nv);
}
#endif  // KDN_PREFILL_VARIANT

#ifdef KDN_PREFILL_DISPATCH
int prefill_value_block(const PrefillParams &P) {
    // Enough workgroups to cover the 256 CUs, value blocks of 16 or 32
    // columns (float32 operands: 16, for the LDS budget).
    if (!P.bf16)
        return 16;
    const long heads = (long)P.B * P.H;
    int nv = 32;
    while (nv > 16 && heads * (P.dv / nv) < 256)
        nv >>= 1;
    return nv;
}

hipError_t launch_prefill(const PrefillParams &P, hipStream_t st) {
    if ((long)P.B * P.H == 0)
        return hipSuccess;
    const int nv = prefill_value_block(P);
    switch (P.variant) {
    case DELTANET: return launch_prefill_v0(P, st, nv);
    case GATED_DELTANET: return launch_prefill_v1(P, st, nv);
    case KDA: return launch_prefill_v2(P, st, nv);
    case DIAG_KDN: return launch_prefill_v3(P, st, nv);
    }
    return hipErrorInvalidValue;
}
#endif  // KDN_PREFILL_DISPATCH

}  // namespace kdn
