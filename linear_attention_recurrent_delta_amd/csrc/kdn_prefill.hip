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
//   1  commit the raw q, k, alpha, xi tiles and the v block (loaded one chunk
//      ahead into registers with 16 B loads) to LDS;
//   2  decay and write vectors: KDN variance chain (one thread per key
//      channel, sequential in t), then a two-level product scan of the decays
//      over token groups with all 256 threads, then the scaled operands K~,
//      Q~, W' = w / gamma and W~^T with 16 B LDS accesses;
//   3  A_kk, A_qk on MFMA from K~ W'^T and Q~ W'^T (exact elementwise
//      fallback when a channel decays below 2^-90 inside the chunk);
//   4  T = (I + A_kk)^-1: 16x16 diagonal blocks by forward substitution (one
//      wave per block), off-diagonal blocks by MFMA block doubling:
//      T[b,a] = -T[b,b] A[b,a] T[a,a] on 16- then 32-row blocks;
//   5  U = V - K~ S on MFMA (overlaps 4's diagonal blocks);
//   6  E = T U on MFMA;
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
    static constexpr int ES = (int)sizeof(E);
    static constexpr int PADE = 16 / ES;
    static constexpr int PK = DK + PADE;     // pitch of [*][DK] operands
    static constexpr int PC = C + PADE;      // pitch of [*][C] operands
    static constexpr int PV = NV + PADE;     // pitch of the staged v block
    static constexpr int PA = C + 4;         // pitch of the fp32 A_kk
    static constexpr int PP = DK + 4;        // pitch of the fp32 KDN u = p- k
    static constexpr int NB = C / 16;        // 16-row blocks per chunk
    static constexpr bool DECAY = VAR != DELTANET;
    static constexpr bool VDECAY = VAR == KDA || VAR == DIAG_KDN;
    static constexpr bool KDN = VAR == DIAG_KDN;
    // row layout of the decay scan: 8 channels x TPG tokens per thread
    static constexpr int NO = DK / 8;        // channel octets
    static constexpr int NG = NT / NO;       // token groups
    static constexpr int TPG = C / NG;       // tokens per group

    static constexpr int SZ_CK = C * PK * ES;
    static constexpr int OFF_KT = 0;
    static constexpr int OFF_QT = OFF_KT + SZ_CK;
    static constexpr int OFF_WP = OFF_QT + SZ_CK;
    static constexpr int OFF_ALP = OFF_WP + SZ_CK;
    static constexpr int OFF_WTT = OFF_ALP + (VDECAY ? SZ_CK : 0);
    static constexpr int SZ_WTT = DK * PC * ES;
    static constexpr int OFF_ST = OFF_WTT + SZ_WTT;
    static constexpr int OFF_VR = OFF_ST + NV * PK * ES;
    // A_kk (then T, in place), A_qk, U^T, E^T; during phase 2 the same bytes
    // hold the KDN u = p- k array and the scan's group products.
    static constexpr int OFF_AKK = OFF_VR + C * PV * ES;
    static constexpr int OFF_AQ = OFF_AKK + C * PA * 4;
    static constexpr int OFF_UT = OFF_AQ + C * PC * ES;
    static constexpr int OFF_ET = OFF_UT + NV * PC * ES;
    static constexpr int END_ET = OFF_ET + NV * PC * ES;
    static constexpr int OFF_U32 = OFF_AKK;
    static constexpr int OFF_GP = OFF_AKK + (KDN ? C * PP * 4 : 0);
    static constexpr int OFF_GS = OFF_GP + NG * DK * 4;
    static constexpr int END_SCAN = OFF_GS + (DECAY ? NG * DK * 4 : 0);
    static constexpr int END_A = END_ET > END_SCAN ? END_ET : END_SCAN;
    // fp32 scratch of the triangular inverse: T[0:32,0:32]^T (pitch 36),
    // T[32:48,32:48]^T (pitch 20) and the transposed block products; in W'
    // (and the raw alpha tile after it, both dead after phase 3) when it
    // fits, else a region of its own
    static constexpr int SZ_T = NB == 4 ? (32 * 36 + 16 * 20 + 32 * 36) * 4
                                        : (16 * 36 + 16 * 20) * 4;
    static constexpr bool T_IN_WP = SZ_T <= SZ_CK * (VDECAY ? 2 : 1);
    static constexpr int OFF_TTA = T_IN_WP ? OFF_WP : END_A;
    static constexpr int OFF_TTB = OFF_TTA + (NB == 4 ? 32 : 16) * 36 * 4;
    static constexpr int OFF_TS = OFF_TTB + (NB == 4 ? 16 * 20 * 4 : 0);
    static constexpr int OFF_SM = T_IN_WP ? END_A : END_A + SZ_T;
    static constexpr int SM_BETA = 0, SM_R = C, SM_ALPH = 2 * C, SM_INVS = 3 * C,
                         SM_GC = 4 * C, SM_FLAG = 4 * C + DK;
    static constexpr int SZ_SM = (4 * C + DK + 4) * 4;
    static constexpr int TOTAL = OFF_SM + SZ_SM;

    static_assert(TOTAL <= 163840, "prefill LDS budget");
    static_assert(!KDN || C * PK <= DK * PC, "xi staging alias");
    static_assert(NG * TPG == C && TPG >= 1 && TPG <= 8, "scan layout");
    static_assert(C % 16 == 0 && NV % 16 == 0 && DK % 16 == 0, "tiles");
    static_assert(NB == 2 || NB == 4, "chunk of 32 or 64");
    static_assert(NT % C == 0, "row reduction layout");
};

// A ROWS x D tile held in registers between its global load and its LDS
// store, so that the next chunk's loads are in flight during this chunk's
// compute.  The loaded registers are not touched until commit() (any use
// would make the wave wait for the load).  Rows t >= L load row L-1 (always
// in bounds, L >= 1) and are replaced by `pad` at commit.
template <typename T, int D, int ROWS>
struct TileRegs {
    static constexpr int VN = 16 / (int)sizeof(T);
    static constexpr int VPR = D / VN;
    static constexpr int NV16 = ROWS * VPR;
    static constexpr int N = (NV16 + 255) / 256;
    static_assert(VPR * VN == D, "row width");
    uint4 r[N];
    int L;

    __device__ __forceinline__ void fetch(const T *src, long stride, int L_,
                                          int tid) {
        L = L_;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int x = tid + 256 * n;
            if (NV16 % 256 == 0 || x < NV16) {
                const int t = x / VPR, c = x % VPR;
                const int tl = t < L_ ? t : L_ - 1;
                r[n] = *reinterpret_cast<const uint4 *>(src + (long)tl * stride + c * VN);
            }
        }
    }
    __device__ __forceinline__ void commit(T *dst, int pitch, float pad,
                                           int tid) const {
        const T pv = from_f32<T>(pad);
        T tmp[VN];
#pragma unroll
        for (int e = 0; e < VN; ++e)
            tmp[e] = pv;
        const uint4 padv = *reinterpret_cast<const uint4 *>(tmp);
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int x = tid + 256 * n;
            if (NV16 % 256 == 0 || x < NV16) {
                const int t = x / VPR, c = x % VPR;
                const bool in = t < L;
                uint4 v;
                v.x = in ? r[n].x : padv.x;
                v.y = in ? r[n].y : padv.y;
                v.z = in ? r[n].z : padv.z;
                v.w = in ? r[n].w : padv.w;
                *reinterpret_cast<uint4 *>(dst + t * pitch + c * VN) = v;
            }
        }
    }
};

// Copy ROWS x D elements straight from global memory into LDS (the exact
// decay path only; rows t >= L get `pad`).
template <typename T, int D, int ROWS>
__device__ __forceinline__ void stage_rows(T *dst, int pitch, const T *src,
                                           long stride, int L, float pad, int tid) {
    TileRegs<T, D, ROWS> t;
    t.fetch(src, stride, L, tid);
    t.commit(dst, pitch, pad, tid);
}

template <typename E>
__device__ __forceinline__ float ld(const E *p) { return to_f32(*p); }

// acc += A[0:16, 0:K] * B[0:K, 0:16] with A read from fp32 LDS rows ([row][k],
// pitch lda) and rounded to the operand type E, B given as [col][k] in E.
template <typename E>
__device__ __forceinline__ void mma_tile_f32a(f32x4 &acc, const float *A, int lda,
                                              const E *B, int ldb, int K, int lane) {
    const int r = lane & 15;
    const int ko = (lane >> 4) * Mma<E>::KPL;
    const float *pa = A + r * lda + ko;
    const E *pb = B + r * ldb + ko;
    for (int k = 0; k < K; k += Mma<E>::KSTEP) {
        if constexpr (sizeof(E) == 2) {
            const float4 a0 = *reinterpret_cast<const float4 *>(pa + k);
            const float4 a1 = *reinterpret_cast<const float4 *>(pa + k + 4);
            bf16x8 av;
            av[0] = static_cast<bf16>(a0.x); av[1] = static_cast<bf16>(a0.y);
            av[2] = static_cast<bf16>(a0.z); av[3] = static_cast<bf16>(a0.w);
            av[4] = static_cast<bf16>(a1.x); av[5] = static_cast<bf16>(a1.y);
            av[6] = static_cast<bf16>(a1.z); av[7] = static_cast<bf16>(a1.w);
            const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(pb + k);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
        } else {
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k], pb[k], acc, 0, 0, 0);
        }
    }
}

template <typename E, int VAR, int DK, int NV, int C>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams P) {
    using LY = PrefillLayout<E, VAR, DK, NV, C>;
    constexpr int PK = LY::PK, PC = LY::PC, PV = LY::PV, PA = LY::PA,
                  PP = LY::PP, NB = LY::NB;
    constexpr int NO = LY::NO, NG = LY::NG, TPG = LY::TPG;
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
    float *U32 = reinterpret_cast<float *>(smem + LY::OFF_U32);   // KDN u
    float *GP = reinterpret_cast<float *>(smem + LY::OFF_GP);     // scan
    float *GS = reinterpret_cast<float *>(smem + LY::OFF_GS);
    E *AQ = reinterpret_cast<E *>(smem + LY::OFF_AQ);
    E *UT = reinterpret_cast<E *>(smem + LY::OFF_UT);
    E *ET = reinterpret_cast<E *>(smem + LY::OFF_ET);
    float *TTA = reinterpret_cast<float *>(smem + LY::OFF_TTA);   // T^T blocks
    float *TTB = reinterpret_cast<float *>(smem + LY::OFF_TTB);
    float *TS = reinterpret_cast<float *>(smem + LY::OFF_TS);     // products
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

    // Raw tiles of the next chunk, in flight while the current one computes.
    TileRegs<E, DK, C> rk, rq, ra, rx;
    TileRegs<E, NV, C> rv;
    E sc_b = from_f32<E>(0.f), sc_r = from_f32<E>(1.f), sc_a = from_f32<E>(1.f);
    auto fetch = [&](int cs) {
        const int Ls = min(C, T - cs);
        const long tk = ((long)b * T + cs) * H + h;
        rk.fetch(gk + tk * DK, sk_, Ls, tid);
        rq.fetch(gq + tk * DK, sk_, Ls, tid);
        if (VDECAY) ra.fetch(ga + tk * DK, sk_, Ls, tid);
        if (KDN) rx.fetch(gx + tk * DK, sk_, Ls, tid);
        rv.fetch(gv + tk * DV + v0, sv_, Ls, tid);
        if (tid < C) {
            const long ti = tk + (long)min(tid, Ls - 1) * H;
            if (!KDN) sc_b = gb[ti]; else sc_r = gr[ti];
            if (VAR == GATED_DELTANET) sc_a = ga[ti];
        }
    };
    if (T > 0)
        fetch(0);

    // scan-layout coordinates: channels i0..i0+7, tokens t0..t0+TPG-1
    const int oc = tid % NO, grp = tid / NO;
    const int i0 = oc * 8, t0 = grp * TPG;

    for (int c0 = 0; c0 < T; c0 += C) {
        const int L = min(C, T - c0);
        const long tok0 = ((long)b * T + c0) * H + h;   // (b, c0, h)

        // ---------------- 1. stage raw tiles ----------------
        rk.commit(Kt, PK, 0.f, tid);
        rq.commit(Qt, PK, 0.f, tid);
        if (VDECAY) ra.commit(ALP, PK, 1.f, tid);
        if (KDN) rx.commit(XR, PK, 0.f, tid);
        rv.commit(VR, PV, 0.f, tid);
        if (tid < C) {
            const bool in = tid < L;
            if (!KDN) s_beta[tid] = in ? to_f32(sc_b) : 0.f;
            else s_r[tid] = in ? to_f32(sc_r) : 1.f;
            if (VAR == GATED_DELTANET) s_alph[tid] = in ? to_f32(sc_a) : 1.f;
        }
        if (tid == 0)
            *s_flag = 0;
        __syncthreads();
        if (c0 + C < T)
            fetch(c0 + C);

        // ---------------- 2. decays and write vectors ----------------
        if constexpr (KDN) {
            // Variance chain, one thread per key channel (sequential in t):
            //   p- = a^2 p + xi,  u = p- k,  p = p- r / (r + mu p- k^2).
            if (tid < DK) {
                const int i = tid;
#pragma unroll 8
                for (int t = 0; t < C; ++t) {
                    const float kk = ld(Kt + t * PK + i);
                    const float a = ld(ALP + t * PK + i);
                    const float x = ld(XR + t * PK + i);
                    const float r = s_r[t];
                    const float pm = a * a * p_reg + x;
                    const float u = pm * kk;
                    U32[t * PP + i] = u;
                    const float den = r + P.mu * pm * kk * kk;
                    if (t < L)
                        p_reg = (den != 0.f) ? pm * r * fast_rcp(den) : pm;
                }
            }
            __syncthreads();
            // innovation variances s_t = r_t + sum_i u_ti k_ti
            constexpr int TPR = 256 / C;          // threads per token row
            constexpr int CPT = DK / TPR;          // channels per thread
            const int t = tid / TPR, part = tid % TPR;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CPT; c += 8) {
                float uu[8], kk[8];
                lds_ld8(U32 + t * PP + part * CPT + c, uu);
                lds_ld8(Kt + t * PK + part * CPT + c, kk);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc += uu[e] * kk[e];
            }
#pragma unroll
            for (int off = TPR / 2; off >= 1; off >>= 1)
                acc += __shfl_xor(acc, off, WAVE);
            if (part == 0) {
                const float s = s_r[t] + acc;
                s_invs[t] = (s != 0.f) ? 1.f / s : 0.f;
            }
        }
        // 2a. in-group products of the decays
        float av[TPG][8], lp[TPG][8];
        if constexpr (DECAY) {
#pragma unroll
            for (int tt = 0; tt < TPG; ++tt) {
                const int t = t0 + tt;
                if constexpr (VDECAY) {
                    lds_ld8(ALP + t * PK + i0, av[tt]);
                } else {
                    const float a = s_alph[t];
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        av[tt][c] = a;
                }
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    lp[tt][c] = tt ? lp[tt - 1][c] * av[tt][c] : av[tt][c];
            }
            lds_st8(GP + grp * DK + i0, lp[TPG - 1]);   // group totals
            __syncthreads();
            // 2b. exclusive prefix / suffix over groups, one thread per channel
            if (tid < DK) {
                float gt[NG];
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    gt[g] = GP[g * DK + tid];
                float pre = 1.f;
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    GP[g * DK + tid] = pre;
                    pre *= gt[g];
                }
                float suf = 1.f;
#pragma unroll
                for (int g = NG - 1; g >= 0; --g) {
                    GS[g * DK + tid] = suf;
                    suf *= gt[g];
                }
                s_gc[tid] = pre;                       // gamma_C of channel
                if (!(pre >= KDN_DECAY_FLOOR))
                    *s_flag = 1;
            }
        }
        __syncthreads();
        // 2c. scaled operands (row layout, 16 B LDS accesses)
        const bool fb = DECAY && (*s_flag != 0);
        {
            float pre[8], suf[8];
            if constexpr (DECAY) {
                lds_ld8(GP + grp * DK + i0, pre);
                lds_ld8(GS + grp * DK + i0, suf);
            }
            float w[TPG][8];
#pragma unroll
            for (int tt = 0; tt < TPG; ++tt) {
                const int t = t0 + tt;
                float kk[8];
                lds_ld8(Kt + t * PK + i0, kk);
                if constexpr (KDN) {
                    float uu[8];
                    lds_ld8(U32 + t * PP + i0, uu);
                    const float inv = s_invs[t];
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        w[tt][c] = uu[c] * inv;
                } else {
                    const float bt = s_beta[t];
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        w[tt][c] = bt * kk[c];
                }
                if constexpr (DECAY) {
                    float qq[8], g[8], o[8];
                    lds_ld8(Qt + t * PK + i0, qq);
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        g[c] = pre[c] * lp[tt][c];
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        o[c] = g[c] * kk[c];
                    lds_st8(Kt + t * PK + i0, o);
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        o[c] = g[c] * qq[c];
                    lds_st8(Qt + t * PK + i0, o);
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        o[c] = fb ? w[tt][c] : w[tt][c] * fast_rcp(g[c]);
                    lds_st8(Wp + t * PK + i0, o);
                } else {
                    lds_st8(Wp + t * PK + i0, w[tt]);
                }
            }
            // W~^T[i][t] = (gamma_C / gamma_t) w_t: suffix products of the
            // group's own tokens times the groups after it
            float wt[8][TPG];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                float sg = DECAY ? suf[c] : 1.f;
#pragma unroll
                for (int tt = TPG - 1; tt >= 0; --tt) {
                    wt[c][tt] = sg * w[tt][c];
                    if (DECAY)
                        sg *= av[tt][c];
                }
            }
#pragma unroll
            for (int c = 0; c < 8; ++c)
                lds_stn<TPG>(WtT + (i0 + c) * PC + t0, wt[c]);
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
                mma_tile_k<E, DK>(acc, (which ? Qt : Kt) + mi * 16 * PK, PK,
                                  Wp + ni * 16 * PK, PK, lane);
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
        // zero the blocks above the diagonal of A_qk and A_kk (T is built in
        // place in A_kk; MFMA K ranges may cover these blocks)
        for (int x = tid; x < C * C; x += 256) {
            const int t = x / C, s = x % C;
            if ((s >> 4) > (t >> 4)) {
                AQ[t * PC + s] = from_f32<E>(0.f);
                Akk[t * PA + s] = 0.f;
            }
        }
        __syncthreads();

        // ---------------- 5. U = V - K~ S  (overlaps 4a) ----------------
        constexpr int NTU = NB * NTJ;
        for (int x = wv; x < NTU; x += 4) {
            const int mi = x / NTJ, nj = x % NTJ;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile_k<E, DK>(acc, Kt + mi * 16 * PK, PK, ST + nj * 16 * PK, PK, lane);
            const int j = nj * 16 + (lane & 15);
            float uo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = mi * 16 + (lane >> 4) * 4 + r;
                uo[r] = ld(VR + t * PV + j) - acc[r];
            }
            lds_stn<4>(UT + j * PC + mi * 16 + (lane >> 4) * 4, uo);
        }
        // ---------------- 4a. diagonal blocks of T ----------------
        // T[I,I] = (I + A[I,I])^-1 by forward substitution, in place in A_kk
        // (fp32); wave I, lane j computes column j.  Row r of the block is
        // read before it is overwritten (LDS operations of a wave are in
        // order).  Transposed copies of the blocks that later products take
        // as B operands go to TTA (blocks 0, 1) and TTB (block 2).
        if (wv < NB && lane < 16) {
            const int o0 = wv * 16, j = lane;
            float xv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m)
                    acc += Akk[(o0 + r) * PA + o0 + m] * xv[m];
                xv[r] = (r == j) ? 1.f : ((r < j) ? 0.f : -acc);
                Akk[(o0 + r) * PA + o0 + j] = xv[r];
            }
            float *dst = wv < 2 ? TTA + (o0 + j) * 36 + o0
                                : (wv == 2 ? TTB + j * 20 : nullptr);
            if (dst) {
#pragma unroll
                for (int r = 0; r < 16; r += 4)
                    *reinterpret_cast<float4 *>(dst + r) =
                        make_float4(xv[r], xv[r + 1], xv[r + 2], xv[r + 3]);
            }
        }
        __syncthreads();
        // ---------------- 4b. off-diagonal blocks of T ----------------
        // 16-row pairs: T[2p+1,2p] = -T[2p+1,2p+1] (A[2p+1,2p] T[2p,2p]).
        {
            constexpr int NPAIR = NB / 2;
            if (wv < NPAIR) {
                const int ra = (2 * wv + 1) * 16, ca = 2 * wv * 16;
                const float *Bt = wv == 0 ? TTA : TTB;          // T[ca,ca]^T
                const int ldb = wv == 0 ? 36 : 20;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                Mma16<float>::tile(acc, Akk + ra * PA + ca, PA, Bt, ldb, lane);
                // P^T[n][k] for the next product's B operand
                *reinterpret_cast<float4 *>(TS + wv * 16 * 20 + (lane & 15) * 20 +
                                            (lane >> 4) * 4) =
                    make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
            __syncthreads();
            if (wv < NPAIR) {
                const int ra = (2 * wv + 1) * 16, ca = 2 * wv * 16;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                Mma16<float>::tile(acc, Akk + ra * PA + ra, PA, TS + wv * 16 * 20, 20, lane);
                const int col = ca + (lane & 15), row0 = ra + (lane >> 4) * 4;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Akk[(row0 + r) * PA + col] = -acc[r];
                if (wv == 0)            // T[1,0]^T joins T[0:32,0:32]^T
                    *reinterpret_cast<float4 *>(TTA + col * 36 + row0) =
                        make_float4(-acc[0], -acc[1], -acc[2], -acc[3]);
            }
            __syncthreads();
        }
        if constexpr (NB == 4) {
            // 32-row halves: T[b,a] = -T[b,b] (A[b,a] T[a,a]), b = rows 32..63,
            // a = rows 0..31; one 16x16 tile (mi, ni) per wave.
            const int mi = wv >> 1, ni = wv & 1;
            {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (kb >= ni)            // T[a] is lower block-triangular
                        Mma16<float>::tile(acc, Akk + (32 + mi * 16) * PA + kb * 16, PA,
                                           TTA + ni * 16 * 36 + kb * 16, 36, lane);
                // Q^T[ni*16 + j][mi*16 + row]
                *reinterpret_cast<float4 *>(TS + (ni * 16 + (lane & 15)) * 36 + mi * 16 +
                                            (lane >> 4) * 4) =
                    make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
            __syncthreads();
            {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (kb <= mi)
                        Mma16<float>::tile(acc, Akk + (32 + mi * 16) * PA + 32 + kb * 16, PA,
                                           TS + ni * 16 * 36 + kb * 16, 36, lane);
                const int col = ni * 16 + (lane & 15), row0 = 32 + mi * 16 + (lane >> 4) * 4;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Akk[(row0 + r) * PA + col] = -acc[r];
            }
            __syncthreads();
        }

        // ---------------- 6. E = T U ----------------
        for (int x = wv; x < NTU; x += 4) {
            const int mi = x / NTJ, nj = x % NTJ;
            const int kc = min(C, ((mi + 1) * 16 + KS - 1) / KS * KS);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile_f32a<E>(acc, Akk + mi * 16 * PA, PA, UT + nj * 16 * PC, PC, kc, lane);
            const int j = nj * 16 + (lane & 15);
            float eo[4] = {acc[0], acc[1], acc[2], acc[3]};
            lds_stn<4>(ET + j * PC + mi * 16 + (lane >> 4) * 4, eo);
        }
        __syncthreads();

        // ---------------- 7. outputs and state ----------------
        E *go = static_cast<E *>(P.o);
        for (int x = wv; x < NTU; x += 4) {
            const int mi = x / NTJ, nj = x % NTJ;
            const int kc = min(C, ((mi + 1) * 16 + KS - 1) / KS * KS);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile_k<E, DK>(acc, Qt + mi * 16 * PK, PK, ST + nj * 16 * PK, PK, lane);
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
            mma_tile_k<E, C>(sacc[u], WtT + ti * 16 * PC, PC, ET + tj * 16 * PC, PC, lane);
        }
        __syncthreads();

        // ---------------- 8. S for the next chunk's products ----------------
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int tau = wv + 4 * u, ti = tau / NTJ, tj = tau % NTJ;
            const int j = tj * 16 + (lane & 15);
            float so[4] = {sacc[u][0], sacc[u][1], sacc[u][2], sacc[u][3]};
            lds_stn<4>(ST + j * PK + ti * 16 + (lane >> 4) * 4, so);
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
