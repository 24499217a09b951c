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
// does not depend on S and runs per channel inside the chunk.  Isotropic KDN
// (same page, section "各向同性近似：把整个头压缩成一个数") is KDA whose write
// strengths beta_t = p-_t / (r_t + p-_t |k_t|^2) come from one variance per
// head; inside a chunk its token maps (Mobius form) are scanned across the
// lanes of one wave.
//
// Two kernels are instantiated from prefill_kernel:
//  - PREP = true, the chunk-parallel prep kernel of the two-pass schedule:
//    persistent 8-wave workgroups, one per CU, each walking every gridDim-th
//    (batch*head, chunk) unit and writing steps 1-4 of the unit to its
//    workspace record (kdn_workspace.h);
//  - PREP = false, the single-pass kernel: one 8-wave workgroup owns one
//    (batch, head, d_v block of NV columns) and walks all chunks in order, the
//    d_k x NV slice of S in MFMA accumulator registers in float32 for the whole
//    sequence.  Sibling workgroups of a head (different d_v blocks) repeat the
//    S-independent work (decay prep, gains, A matrices, triangular inverse) so
//    that the grid fills the CUs; they are placed on one XCD so that q/k/gate
//    reads hit its L2.
//
// Per chunk:
//   1  commit the raw q, k, alpha, xi tiles and the v block (loaded one chunk
//      ahead into registers with 16 B loads) to LDS;
//   2  decay and write vectors: KDN variance chain (one thread per key
//      channel, sequential in t), then a two-level product scan of the decays
//      over token groups (256 threads), then the scaled operands K~,
//      Q~, W' = w / gamma and W~^T with 16 B LDS accesses;
//   3  A_kk, A_qk on MFMA from K~ W'^T and Q~ W'^T (exact elementwise
//      fallback when a channel decays below 2^-90 inside the chunk);
//   4  T = (I + A_kk)^-1: each 16x16 diagonal block by one wave (two 8x8
//      forward substitutions and one 8x8 product); the blocks below the
//      diagonal on (near) fp32 MFMA -- in the prep kernel from the
//      factorisation I + A = (I + N D) D^-1 (D the inverted diagonal blocks,
//      N the blocks below the diagonal) in three levels of independent block
//      products, in the single-pass kernel one chain per block column,
//      T[I,J] = -T[I,I] sum_K A[I,K] T[K,J];
//   5  U = V - K~ S on MFMA (overlaps 4's diagonal blocks);
//   6  E = T U on MFMA;
//   7  O = Q~ S + A_qk E (stored), S = gamma_C S + W~^T E on MFMA;
//   8  S rounded to the operand type for the next chunk's products.
#include "kdn_device.h"
#include "kdn_launch.h"
#include "kdn_workspace.h"

namespace kdn {

#ifdef KDN_PREFILL_VARIANT
// Below this cumulative in-chunk decay the 1/gamma operand scaling is not
// used (it would leave the float range); the chunk takes the exact path.
#define KDN_DECAY_FLOOR 8.077935669463161e-28f   /* 2^-90 */

template <typename E, int VAR, int DK, int NV, int C, int NW>
struct PrefillLayout {
    static constexpr int NT = 64 * NW;       // threads per workgroup
    static constexpr int ES = (int)sizeof(E);
    static constexpr int PADE = 16 / ES;
    static constexpr int PK = DK + PADE;     // pitch of [*][DK] operands
    static constexpr int PC = C + PADE;      // pitch of [*][C] operands
    static constexpr int PV = NV + PADE;     // pitch of the staged v block
    static constexpr int PA = C + 4;         // pitch of the fp32 A_kk
    static constexpr int PP = DK + 4;        // pitch of the fp32 KDN u = p- k
    static constexpr int NB = C / 16;        // 16-row blocks per chunk
    static constexpr bool DECAY = VAR != DELTANET;
    static constexpr bool VDECAY = VAR == KDA || VAR == DIAG_KDN || VAR == ISO_KDN;
    static constexpr bool KDN = VAR == DIAG_KDN;
    static constexpr bool ISO = VAR == ISO_KDN;
    // row layout of the decay scan: 8 channels x TPG tokens per thread
    static constexpr int NO = DK / 8;        // channel octets
    static constexpr int NG = 256 / NO < C ? 256 / NO : C; // token groups
    static constexpr int NTS = NO * NG;      // threads of the scan layout
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
    // T in the operand type for E = T U
    static constexpr int OFF_TM = END_A;
    static constexpr int END_TM = OFF_TM + C * PC * ES;
    // fp32 scratch of the triangular inverse (16 x 20 blocks): T[I,I] for
    // all I, T[I,I]^T for I < NB-1, then per column-chain wave J the
    // products P^T and T[K,J]^T (K = J+1 .. NB-2); in W' (and the alpha tile after it,
    // both dead after phase 3) when it fits, else a region of its own
    static constexpr int NSLOT = NB + (NB - 1) + (NB - 1) * NB / 2;
    static constexpr int SZ_T = NSLOT * 16 * 20 * 4;
    static constexpr bool T_IN_WP = SZ_T <= SZ_CK * (VDECAY ? 2 : 1);
    static constexpr int OFF_TD = T_IN_WP ? OFF_WP : END_TM;
    static constexpr int OFF_SM = T_IN_WP ? END_TM : END_TM + SZ_T;
    static constexpr int SM_BETA = 0, SM_R = C, SM_ALPH = 2 * C, SM_INVS = 3 * C,
                         SM_GC = 4 * C, SM_FLAG = 4 * C + DK, SM_WSC = 4 * C + DK + 4,
                         SM_ZR = 5 * C + DK + 4;
    static constexpr int SZ_SM = (6 * C + DK + 4) * 4;
    static constexpr int TOTAL = OFF_SM + SZ_SM;

    static_assert(TOTAL <= 163840, "prefill LDS budget");
    static_assert(!(KDN || ISO) || C * PK <= DK * PC, "xi staging alias");
    static_assert(NG * TPG == C && TPG >= 1 && TPG <= 8, "scan layout");
    static_assert(C % 16 == 0 && NV % 16 == 0 && DK % 16 == 0, "tiles");
    static_assert(NB == 2 || NB == 4, "chunk of 32 or 64");
    static_assert(NT % C == 0, "row reduction layout");
    // KDN innovation sums: TPR threads per token row, 8k channels each
    static constexpr int TPR = (NT / C) < (DK / 8) ? (NT / C) : (DK / 8);
};

// A ROWS x D tile held in registers between its global load and its LDS
// store, so that the next chunk's loads are in flight during this chunk's
// compute.  The loaded registers are not touched until commit() (any use
// would make the wave wait for the load).  Rows t >= L load row L-1 (always
// in bounds, L >= 1) and are replaced by `pad` at commit.
template <typename T, int D, int ROWS, int NT>
struct TileRegs {
    static constexpr int VN = 16 / (int)sizeof(T);
    static constexpr int VPR = D / VN;
    static constexpr int NV16 = ROWS * VPR;
    static constexpr int N = (NV16 + NT - 1) / NT;
    static_assert(VPR * VN == D, "row width");
    uint4 r[N];
    int L;

    __device__ __forceinline__ void fetch(const T *src, long stride, int L_,
                                          int tid) {
        L = L_;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int x = tid + NT * n;
            if (NV16 % NT == 0 || x < NV16) {
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
            const int x = tid + NT * n;
            if (NV16 % NT == 0 || x < NV16) {
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
template <typename T, int D, int ROWS, int NT>
__device__ __forceinline__ void stage_rows(T *dst, int pitch, const T *src,
                                           long stride, int L, float pad, int tid) {
    TileRegs<T, D, ROWS, NT> t;
    t.fetch(src, stride, L, tid);
    t.commit(dst, pitch, pad, tid);
}

template <typename E>
__device__ __forceinline__ float ld(const E *p) { return to_f32(*p); }

// acc += A[0:16, 0:16] * B[0:16, 0:16] in (near) fp32: A from fp32 LDS rows
// ([row][k], pitch lda), B from fp32 LDS as [col][k] (pitch ldb).  For bf16
// kernels each operand is split into hi + lo bf16 parts and the three
// significant partial products run on bf16 MFMA; float kernels use the fp32
// MFMA.
template <typename E>
__device__ __forceinline__ void mma16_f32(f32x4 &acc, const float *A, int lda,
                                          const float *B, int ldb, int lane) {
    if constexpr (sizeof(E) == 2) {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const int r = lane & 15, ko = (lane >> 4) * 4;
        const float4 a = *reinterpret_cast<const float4 *>(A + r * lda + ko);
        const float4 b = *reinterpret_cast<const float4 *>(B + r * ldb + ko);
        const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
        bf16x4 ah, al, bh, bl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ah[e] = static_cast<bf16>(av[e]);
            al[e] = static_cast<bf16>(av[e] - static_cast<float>(ah[e]));
            bh[e] = static_cast<bf16>(bv[e]);
            bl[e] = static_cast<bf16>(bv[e] - static_cast<float>(bh[e]));
        }
        const s16x4 ahs = *reinterpret_cast<const s16x4 *>(&ah);
        const s16x4 als = *reinterpret_cast<const s16x4 *>(&al);
        const s16x4 bhs = *reinterpret_cast<const s16x4 *>(&bh);
        const s16x4 bls = *reinterpret_cast<const s16x4 *>(&bl);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(als, bhs, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahs, bls, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahs, bhs, acc, 0, 0, 0);
    } else {
        Mma16<float>::tile(acc, A, lda, B, ldb, lane);
    }
}

// Records are written once and read once, by another kernel: their stores
// are non-temporal, so that they do not push the prep kernel's own tiles out
// of L2 (measured: every two-pass prefill about 4 % faster).
__device__ __forceinline__ void store_rec16(uint4 *d, uint4 v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(d));
}

// A-operand fragment order of the workspace (kdn_workspace.h): copy the
// R x K matrix at src (LDS, pitch in elements) to dst, 16 bytes per unit;
// with perm (bf16), the columns of each 32-group in the permuted order, and
// with neg (bf16) every element negated (sign bit flipped, exact).
template <typename E, int R, int K, int NT>
__device__ __forceinline__ void store_frag(char *dst, const E *src, int pitch, int tid,
                                           bool perm, bool neg = false) {
    constexpr int EPU = 16 / (int)sizeof(E);
    constexpr int KG = sizeof(E) == 2 ? 32 : 16;
    constexpr int NU = R * K / EPU;
    static_assert(K % KG == 0 && R % 16 == 0, "fragment tiling");
    uint4 *d = reinterpret_cast<uint4 *>(dst);
#pragma unroll
    for (int u0 = 0; u0 < NU; u0 += NT) {
        const int u = u0 + tid;
        if (NU % NT == 0 || u < NU) {
            const int l = u & 63, grp = u >> 6;
            const int m = grp / (K / KG), g = grp % (K / KG);
            const int row = m * 16 + (l & 15);
            uint4 val;
            if constexpr (sizeof(E) == 2) {
                if (perm) {
                    const E *sp = src + row * pitch + g * 32 + (l >> 4) * 4;
                    const uint2 lo = *reinterpret_cast<const uint2 *>(sp);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(sp + 16);
                    val = make_uint4(lo.x, lo.y, hi.x, hi.y);
                } else {
                    val = *reinterpret_cast<const uint4 *>(src + row * pitch + g * 32 + (l >> 4) * 8);
                }
                const unsigned flip = neg ? 0x80008000u : 0u;
                val = make_uint4(val.x ^ flip, val.y ^ flip, val.z ^ flip, val.w ^ flip);
            } else {
                const float *sp = reinterpret_cast<const float *>(src) + row * pitch + g * 16 + (l >> 4);
                val = __builtin_bit_cast(uint4, make_float4(sp[0], sp[4], sp[8], sp[12]));
            }
            store_rec16(d + u, val);
        }
    }
}

// As store_frag, each element computed by f(row, k) (a float).
template <typename E, int R, int K, int NT, typename F>
__device__ __forceinline__ void store_frag_fn(char *dst, int tid, bool perm, F f) {
    constexpr int EPU = 16 / (int)sizeof(E);
    constexpr int KG = sizeof(E) == 2 ? 32 : 16;
    constexpr int NU = R * K / EPU;
    uint4 *d = reinterpret_cast<uint4 *>(dst);
#pragma unroll
    for (int u0 = 0; u0 < NU; u0 += NT) {
        const int u = u0 + tid;
        if (NU % NT == 0 || u < NU) {
            const int l = u & 63, grp = u >> 6;
            const int m = grp / (K / KG), g = grp % (K / KG);
            const int row = m * 16 + (l & 15);
            E v[EPU];
#pragma unroll
            for (int e = 0; e < EPU; ++e) {
                const int k = sizeof(E) == 2
                                  ? (perm ? perm_col(g, l >> 4, e) : g * 32 + (l >> 4) * 8 + e)
                                  : g * 16 + e * 4 + (l >> 4);
                v[e] = from_f32<E>(f(row, k));
            }
            store_rec16(d + u, *reinterpret_cast<const uint4 *>(v));
        }
    }
}

// PREP = false: the single-pass kernel, one workgroup per (batch*head, value
// block) walking all chunks.  PREP = true: the prep kernel of the two-pass
// schedule, one workgroup per (batch*head, chunk): steps 1-4 only, results to
// the workspace record of the chunk.
template <typename E, int VAR, int DK, int NV, int C, int NW, bool PREP>
__global__ __launch_bounds__(64 * NW) void prefill_kernel(PrefillParams P) {
    using LY = PrefillLayout<E, VAR, DK, NV, C, NW>;
    constexpr int NT = LY::NT;
    constexpr int PK = LY::PK, PC = LY::PC, PV = LY::PV, PA = LY::PA,
                  PP = LY::PP, NB = LY::NB;
    constexpr int NO = LY::NO, NG = LY::NG, TPG = LY::TPG;
    constexpr bool DECAY = LY::DECAY, VDECAY = LY::VDECAY, KDN = LY::KDN, ISO = LY::ISO;
    // raw xi tile staged in LDS (the isotropic prep kernel reads per-token
    // sums from the workspace instead)
    constexpr bool XSTAGE = KDN || (ISO && !PREP);
    // Prep kernel, scalar decay: no per-channel scan; the decay enters as
    // ratios gamma_t / gamma_s in log2 form (section 2s below).
    constexpr bool SPREP = PREP && VAR == GATED_DELTANET;
    constexpr int NTJ = NV / 16;                // value tiles
    constexpr int NTI = DK / 16;                // key tiles
    constexpr int NST = NTI * NTJ;              // S tiles
    constexpr int NS = (NST + NW - 1) / NW;     // S tiles per wave (max)
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
    E *Tm = reinterpret_cast<E *>(smem + LY::OFF_TM);             // T
    float *TD = reinterpret_cast<float *>(smem + LY::OFF_TD);     // T scratch
    float *sm = reinterpret_cast<float *>(smem + LY::OFF_SM);
    float *s_beta = sm + LY::SM_BETA, *s_r = sm + LY::SM_R,
          *s_alph = sm + LY::SM_ALPH, *s_invs = sm + LY::SM_INVS,
          *s_gc = sm + LY::SM_GC;
    int *s_flag = reinterpret_cast<int *>(sm + LY::SM_FLAG);
    // isotropic KDN per-token sums: mean a^2, mean xi, |k|^2 (r in s_r)
    float *s_ia2 = s_alph, *s_ixm = s_invs, *s_ikk = sm + LY::SM_WSC;
    float *s_gl = s_r;                 // SPREP: log2 gamma over nonzero decays
    float *s_gt = s_invs;              // SPREP: gamma_t
    float *s_wsc = sm + LY::SM_WSC;    // SPREP: beta_s gamma_C / gamma_s
    int *s_zr = reinterpret_cast<int *>(sm + LY::SM_ZR);   // SPREP: last zero decay <= t

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    // records in the permuted column order (bf16 chain kernel)
    const bool perm = sizeof(E) == 2 && P.rec_perm != 0;

    // Workgroup -> (batch*head, value block).  Dispatch is round-robin over
    // the 8 XCDs; place the value blocks of one head on one XCD.
    // PREP: persistent workgroups; unit u = (batch*head, chunk) = divmod(u, NC)
    // for u = blockIdx.x, blockIdx.x + gridDim.x, ...
    const int T = P.T, H = P.H, DV = P.dv;
    const int NC = (T + C - 1) / C;
    const int NU = P.B * H * NC;
    int bh, vb, cbeg;
    if constexpr (PREP) {
        bh = blockIdx.x / NC;
        cbeg = (blockIdx.x % NC) * C;
        vb = 0;
    } else {
        const int nvb = P.dv / NV;
        const int G = gridDim.x;
        int lid = blockIdx.x;
        if ((G & 7) == 0 && ((G >> 3) % nvb) == 0)
            lid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
        bh = lid / nvb;
        vb = lid % nvb;
        cbeg = 0;
    }
    int b = bh / P.H, h = bh % P.H;
    const int v0 = vb * NV;

    const E *gq = static_cast<const E *>(P.q);
    const E *gk = static_cast<const E *>(P.k);
    const E *gv = static_cast<const E *>(P.v);
    const E *ga = static_cast<const E *>(P.alpha);
    const E *gb = static_cast<const E *>(P.beta);
    const E *gx = static_cast<const E *>(P.xi);
    const E *gr = static_cast<const E *>(P.r);

    // ---- S slice in accumulator layout: tile u of this wave is
    //      (ti, tj) = divmod(wv + NW u, NTJ); acc[r] = S[ti*16 + (lane>>4)*4 + r]
    //                                                 [tj*16 + (lane&15)].
    f32x4 sacc[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int tau = wv + NW * u, ti = tau / NTJ, tj = tau % NTJ;
        if (PREP || (NST % NW != 0 && tau >= NST)) continue;
        const int j = tj * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ti * 16 + (lane >> 4) * 4 + r;
            sacc[u][r] = P.S0 ? P.S0[((long)bh * DK + i) * DV + v0 + j] : 0.f;
            ST[j * PK + i] = from_f32<E>(sacc[u][r]);
        }
    }
    float p_reg = 0.f;                 // KDN variance of channel tid (isotropic:
                                       // of the head, in wave 0)
    float p_nxt = 0.f;                 // PREP: variance at the next unit's start
    // Diagonal-KDN prep: thread (s, i) = (tid / DK, tid % DK) runs the
    // variance chain of key channel i over token segment s of the chunk
    // (VLEN tokens), starting from the chunk-start variance pushed through
    // the segment's prefix map (identity for s = 0).
    constexpr int VNS = WsLayout::var_segments(DK);
    constexpr int VLEN = PREP ? C / VNS : C;
    static_assert(!(PREP && KDN) || (VNS * DK == NT && C % VNS == 0), "variance segments");
    float4 q_nxt = make_float4(1.f, 0.f, 0.f, 1.f);
    if (KDN && tid < DK && !PREP)
        p_reg = P.p0[(long)bh * DK + tid];
    if (ISO && tid < WAVE && !PREP)
        p_reg = P.p0[bh];

    const long sk_ = (long)H * DK;     // token stride of q/k/alpha/xi
    const long sv_ = (long)H * DV;     // token stride of v/o

    // Raw tiles of the next chunk, in flight while the current one computes.
    TileRegs<E, DK, C, NT> rk, rq, ra, rx;
    TileRegs<E, NV, C, NT> rv;
    E sc_b = from_f32<E>(0.f), sc_r = from_f32<E>(1.f), sc_a = from_f32<E>(1.f);
    float4 sc_st = make_float4(1.f, 0.f, 0.f, 1.f);   // isotropic prep: token sums
    auto fetch = [&](int bs, int cs) {
        const int Ls = min(C, T - cs);
        const long tk = ((long)(bs / H) * T + cs) * H + bs % H;
        if (PREP && KDN) {
            const long u = (long)bs * NC + cs / C;
            p_nxt = P.ws_p0[u * DK + tid % DK];
            if (tid >= DK)
                q_nxt = reinterpret_cast<const float4 *>(P.ws_pre)[
                    (u * (VNS - 1) + tid / DK - 1) * DK + pre_pos(tid % DK, (int)(16 / sizeof(E)), DK)];
        }
        if (PREP && ISO && tid < WAVE)
            p_nxt = P.ws_p0[(long)bs * NC + cs / C];
        rk.fetch(gk + tk * DK, sk_, Ls, tid);
        rq.fetch(gq + tk * DK, sk_, Ls, tid);
        if (VDECAY) ra.fetch(ga + tk * DK, sk_, Ls, tid);
        if (XSTAGE) rx.fetch(gx + tk * DK, sk_, Ls, tid);
        if (!PREP) rv.fetch(gv + tk * DV + v0, sv_, Ls, tid);
        if (tid < C) {
            const long ti = tk + (long)min(tid, Ls - 1) * H;
            if (ISO && PREP)
                sc_st = reinterpret_cast<const float4 *>(P.ws_stat)[
                    ((long)bs * NC + cs / C) * C + min(tid, Ls - 1)];
            else if (KDN || ISO)
                sc_r = gr[ti];
            else
                sc_b = gb[ti];
            if (VAR == GATED_DELTANET) sc_a = ga[ti];
        }
    };
    if (T > 0 && (!PREP || (int)blockIdx.x < NU))
        fetch(bh, cbeg);

    // Scan layout (threads < NTS): channels i0..i0+7, tokens t0..t0+TPG-1,
    // token groups vary fastest across lanes.  The operand pass uses every
    // thread: H2 threads per group, TPG2 tokens each.
    constexpr int H2 = (NT / LY::NTS) < TPG ? (NT / LY::NTS) : TPG;
    constexpr int TPG2 = TPG / H2, NG2 = NG * H2, NTO = LY::NTS * H2;
    static_assert(TPG2 * H2 == TPG && NTO <= NT, "operand layout");
    // The single-pass diagonal-KDN kernel runs the scan layout on the last
    // NTS threads, alongside the variance chain on the first DK (phase 2).
    // In the prep every thread runs a variance chain; the scan layout is on
    // the first NTS threads, whose waves pass the next unit's loads first.
    static_assert(!(KDN && !PREP) || LY::NTS <= NT - DK, "scan threads clear of the variance chain");
    static_assert(!ISO || LY::NTS <= NT - WAVE, "scan threads clear of wave 0");
    const int ts = ((KDN && !PREP) || ISO) ? tid - (NT - LY::NTS) : tid;   // scan-layout thread, if >= 0
    const int grp = ts % NG, oc = (ts / NG) % NO;
    const int i0 = oc * 8, t0 = grp * TPG;
    const int gh = tid % NG2, oc2 = tid / NG2;
    const int j0 = oc2 * 8, u0 = gh * TPG2;        // operand pass: channels, tokens
    const int ug0 = (gh / H2) * TPG;               // first token of its group

    // 2a. group products of the decays (scan-layout threads): the product of
    // each thread's TPG tokens, per channel
    auto group_products = [&]() {
        float gprod[8];
#pragma unroll
        for (int tt = 0; tt < TPG; ++tt) {
            float a8[8];
            if constexpr (VDECAY) {
                lds_ld8(ALP + (t0 + tt) * PK + i0, a8);
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    a8[c] = s_alph[t0 + tt];
            }
#pragma unroll
            for (int c = 0; c < 8; ++c)
                gprod[c] = tt ? gprod[c] * a8[c] : a8[c];
        }
        lds_st8(GP + grp * DK + i0, gprod);   // group totals
    };

    for (int it = PREP ? (int)blockIdx.x : 0; it < (PREP ? NU : T);
         it += PREP ? (int)gridDim.x : C) {
        int c0 = it;
        if constexpr (PREP) {
            bh = it / NC;
            c0 = (it % NC) * C;
            b = bh / H;
            h = bh % H;
            p_reg = p_nxt;
            if (KDN && tid >= DK)        // variance at the segment start
                p_reg = fmaf(q_nxt.x, p_reg, q_nxt.y) / fmaf(q_nxt.z, p_reg, q_nxt.w);
        }
        const int L = min(C, T - c0);
        const long tok0 = ((long)b * T + c0) * H + h;   // (b, c0, h)

        // ---------------- 1. stage raw tiles ----------------
        rk.commit(Kt, PK, 0.f, tid);
        rq.commit(Qt, PK, 0.f, tid);
        if (VDECAY) ra.commit(ALP, PK, 1.f, tid);
        if (XSTAGE) rx.commit(XR, PK, 0.f, tid);
        if (!PREP) rv.commit(VR, PV, 0.f, tid);
        if (tid < C) {
            // tokens past the end: beta = 0; KDN: a = 1, xi = 0, k = 0, r = 1,
            // which leaves the variance unchanged
            const bool in = tid < L;
            if (ISO && PREP) {
                s_ia2[tid] = in ? sc_st.x : 1.f;
                s_ixm[tid] = in ? sc_st.y : 0.f;
                s_ikk[tid] = in ? sc_st.z : 0.f;
                s_r[tid] = in ? sc_st.w : 1.f;
            } else if (KDN || ISO) {
                s_r[tid] = in ? to_f32(sc_r) : 1.f;
            } else {
                s_beta[tid] = in ? to_f32(sc_b) : 0.f;
            }
            if (VAR == GATED_DELTANET) s_alph[tid] = in ? to_f32(sc_a) : 1.f;
        }
        if (tid == 0)
            *s_flag = 0;
        __syncthreads();
        if (PREP) {
            const int nu = it + (int)gridDim.x;
            if (nu < NU)
                fetch(nu / NC, (nu % NC) * C);
        } else if (c0 + C < T) {
            fetch(bh, c0 + C);
        }

        // ---------------- 2. decays and write vectors ----------------
        if constexpr (KDN) {
            // Variance chain, sequential in t per key channel:
            //   p- = a^2 p + xi,  u = p- k,  p = p- r / (r + mu p- k^2).
            // Single pass: one thread per channel over the whole chunk.  Prep:
            // one thread per (token segment, channel), each from its segment's
            // start variance, so the dependent chain is VLEN steps long.
            // The inputs of a block of CB tokens are read into registers one
            // block ahead; the scheduling barrier keeps those LDS reads at the
            // top of the block, so the dependent chain never waits on LDS.
            // Tokens past the end of the sequence were staged as a = 1,
            // xi = 0, k = 0, r = 1, which leaves p unchanged bit for bit.
            if (ts >= 0 && ts < LY::NTS)
                group_products();          // decays, independent of the variance
            if (PREP || tid < DK) {
                const int i = tid % DK, t0v = (tid / DK) * VLEN, t1v = t0v + VLEN;
                const float mu = P.mu;
                float pc = p_reg;
                constexpr int CB = VLEN < 8 ? VLEN : 8;   // tokens per block
                static_assert(VLEN % CB == 0, "variance blocks");
                float kk[CB], aa[CB], xx[CB], rr[CB];
                auto loadb = [&](int tb) {
#pragma unroll
                    for (int j = 0; j < CB; ++j) {
                        kk[j] = ld(Kt + (tb + j) * PK + i);
                        aa[j] = ld(ALP + (tb + j) * PK + i);
                        xx[j] = ld(XR + (tb + j) * PK + i);
                        rr[j] = s_r[tb + j];
                    }
                };
                loadb(t0v);
#pragma unroll 1
                for (int tb = t0v; tb < t1v; tb += CB) {
                    float a2[CB], x8[CB], m8[CB], k8[CB], r8[CB];
#pragma unroll
                    for (int j = 0; j < CB; ++j) {
                        a2[j] = aa[j] * aa[j];
                        m8[j] = mu * kk[j] * kk[j];
                        x8[j] = xx[j]; k8[j] = kk[j]; r8[j] = rr[j];
                    }
                    // next block (the last block re-reads itself, unused)
                    loadb(min(tb + CB, t1v - CB));
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < CB; ++j) {
                        const float pm = fmaf(a2[j], pc, x8[j]);
                        U32[(tb + j) * PP + i] = pm * k8[j];
                        const float den = fmaf(m8[j], pm, r8[j]);
                        pc = (den != 0.f) ? pm * r8[j] * fast_rcp(den) : pm;
                    }
                }
                p_reg = pc;
            }
            __syncthreads();
            // innovation variances s_t = r_t + sum_i u_ti k_ti
            constexpr int TPR = LY::TPR;           // threads per token row
            constexpr int CPT = DK / TPR;          // channels per thread
            const int t = tid / TPR, part = tid % TPR;
            float acc = 0.f;
            if (tid < TPR * C) {
#pragma unroll
            for (int c = 0; c < CPT; c += 8) {
                float uu[8], kk[8];
                lds_ld8(U32 + t * PP + part * CPT + c, uu);
                lds_ld8(Kt + t * PK + part * CPT + c, kk);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc += uu[e] * kk[e];
            }
            }
#pragma unroll
            for (int off = TPR / 2; off >= 1; off >>= 1)
                acc += __shfl_xor(acc, off, WAVE);
            if (tid < TPR * C && part == 0) {
                const float s = s_r[t] + acc;
                const float invs = (s != 0.f) ? 1.f / s : 0.f;
                s_invs[t] = invs;
                if (PREP && P.invs_out && t < L)     // for the gradient pass
                    P.invs_out[tok0 + (long)t * H] = invs;
            }
        }
        if constexpr (ISO) {
            if constexpr (!PREP) {
                // per-token channel sums: mean a^2, mean xi, |k|^2
                constexpr int TPR = LY::TPR, CPT = DK / TPR;
                const int t = tid / TPR, part = tid % TPR;
                float sa = 0.f, sx = 0.f, sk = 0.f;
                if (tid < TPR * C) {
#pragma unroll
                    for (int c = 0; c < CPT; c += 8) {
                        float a8[8], x8[8], k8[8];
                        lds_ld8(ALP + t * PK + part * CPT + c, a8);
                        lds_ld8(XR + t * PK + part * CPT + c, x8);
                        lds_ld8(Kt + t * PK + part * CPT + c, k8);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            sa = fmaf(a8[e], a8[e], sa);
                            sx += x8[e];
                            sk = fmaf(k8[e], k8[e], sk);
                        }
                    }
                }
#pragma unroll
                for (int off = TPR / 2; off >= 1; off >>= 1) {
                    sa += __shfl_xor(sa, off, WAVE);
                    sx += __shfl_xor(sx, off, WAVE);
                    sk += __shfl_xor(sk, off, WAVE);
                }
                if (tid < TPR * C && part == 0) {
                    s_ia2[t] = sa * (1.f / DK);
                    s_ixm[t] = sx * (1.f / DK);
                    s_ikk[t] = sk;
                }
                __syncthreads();
            }
            if (ts >= 0)
                group_products();          // decays, independent of the variance
            if (wv == 0) {
                // Head variance through the chunk: lane t forms token t's map
                // (predict, then the update with gain numerator (mu/d_k)|k|^2),
                // an inclusive scan over the lanes composes maps 0..t, and the
                // chunk-start variance gives p after every token.  Then
                //   p-_t = mean(a^2) p_{t-1} + mean(xi),
                //   beta_t = p-_t / (r_t + p-_t |k_t|^2)   (0 if that is 0).
                const int t = lane;
                const bool tc = t < C;
                const float a2 = tc ? s_ia2[t] : 1.f, xm = tc ? s_ixm[t] : 0.f;
                const float kk = tc ? s_ikk[t] : 0.f, rt = tc ? s_r[t] : 1.f;
                Map2 m = variance_step_map(a2, xm, P.mu * (1.f / DK) * kk, rt);
                m.rescale();
#pragma unroll
                for (int off = 1; off < C; off <<= 1) {
                    const float ya = __shfl_up(m.a, off, WAVE), yb = __shfl_up(m.b, off, WAVE);
                    const float yc = __shfl_up(m.c, off, WAVE), yd = __shfl_up(m.d, off, WAVE);
                    if (lane >= off) {
                        m.before(ya, yb, yc, yd);
                        m.rescale();
                    }
                }
                const float pt = m.apply(p_reg);          // p after token t
                float pp = __shfl_up(pt, 1, WAVE);        // p after token t - 1
                if (lane == 0)
                    pp = p_reg;
                const float pm = fmaf(a2, pp, xm);
                const float sv = fmaf(pm, kk, rt);
                const float bt = (t < L && sv != 0.f) ? pm / sv : 0.f;
                if (tc)
                    s_beta[t] = bt;
                if (PREP && P.beta_out && t < L)      // for the gradient pass
                    P.beta_out[tok0 + (long)t * H] = bt;
                p_reg = __shfl(pt, C - 1, WAVE);
            }
            __syncthreads();
        }
        bool fb = false;
        // SPREP: raw A-matrix tiles of waves 1.. (tile x = wv-1 + k(NW-1)),
        // computed while wave 0 scans the decays
        constexpr int NL = NB * (NB + 1) / 2;
        constexpr int SPT = SPREP ? (2 * NL + NW - 2) / (NW - 1) : 1;
        f32x4 spacc[SPT];
        if constexpr (SPREP) {
            // 2s. scalar decay: one wave scans log2(alpha_t) over the chunk
            // (zeros tracked separately: the ratio gamma_t / gamma_s is 0 when a
            // zero decay lies in (s, t], else 2^(G_t - G_s)).  The other waves
            // meanwhile form K K^T and Q K^T on MFMA.
            if (wv != 0) {
#pragma unroll
                for (int k = 0; k < SPT; ++k) {
                    const int x = wv - 1 + k * (NW - 1);
                    if (x >= 2 * NL) continue;
                    const int which = x >= NL;
                    int idx = x - which * NL, mi = 0;
                    while (idx > mi) { idx -= mi + 1; ++mi; }
                    spacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
                    mma_tile_k<E, DK>(spacc[k], (which ? Qt : Kt) + mi * 16 * PK, PK,
                                      Kt + idx * 16 * PK, PK, lane);
                }
            }
            if (wv == 0) {
                const int t = lane;
                const float a = t < C ? s_alph[t] : 1.f;
                float gl = a > 0.f ? __builtin_amdgcn_logf(a) : 0.f;
                int zr = a > 0.f ? -1 : t;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float g2 = __shfl_up(gl, off, WAVE);
                    const int z2 = __shfl_up(zr, off, WAVE);
                    if (lane >= off) {
                        gl += g2;
                        zr = max(zr, z2);
                    }
                }
                const float glc = __shfl(gl, C - 1, WAVE);
                const int zrc = __shfl(zr, C - 1, WAVE);
                if (t < C) {
                    s_gl[t] = gl;
                    s_zr[t] = zr;
                    s_gt[t] = zr >= 0 ? 0.f : __builtin_amdgcn_exp2f(gl);
                    s_wsc[t] = zrc > t ? 0.f : s_beta[t] * __builtin_amdgcn_exp2f(glc - gl);
                }
                const float gc = zrc >= 0 ? 0.f : __builtin_amdgcn_exp2f(glc);
                for (int i = lane; i < DK; i += WAVE)
                    s_gc[i] = gc;
            }
            __syncthreads();
        } else {
        // 2a. group products of the decays (KDN: done with the variance above)
        if constexpr (DECAY) {
            if constexpr (!KDN && !ISO) {
                if (ts < LY::NTS)
                    group_products();
                __syncthreads();
            }
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
        // 2c. scaled operands, every thread: channels j0..j0+7, tokens
        //     u0..u0+TPG2-1 (tokens vary fastest across lanes: 16 B row
        //     accesses and the transposed W~ stores stay conflict-free)
        fb = DECAY && (*s_flag != 0);
        if (tid < NTO) {
            const int g = gh / H2;
            float pre[8], suf[8], a8[TPG][8];
            if constexpr (DECAY) {
                lds_ld8(GP + g * DK + j0, pre);
                lds_ld8(GS + g * DK + j0, suf);
#pragma unroll
                for (int tt = 0; tt < TPG; ++tt) {
                    if constexpr (VDECAY) {
                        lds_ld8(ALP + (ug0 + tt) * PK + j0, a8[tt]);
                    } else {
#pragma unroll
                        for (int c = 0; c < 8; ++c)
                            a8[tt][c] = s_alph[ug0 + tt];
                    }
                }
                // in-group tokens before / after this thread's tokens
#pragma unroll
                for (int tt = 0; tt < TPG; ++tt)
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        if (ug0 + tt < u0) pre[c] *= a8[tt][c];
                        if (ug0 + tt >= u0 + TPG2) suf[c] *= a8[tt][c];
                    }
            }
            float w[TPG2][8], ap[TPG2][8];
#pragma unroll
            for (int tt = 0; tt < TPG2; ++tt) {
                const int t = u0 + tt;
                float kk[8];
                lds_ld8(Kt + t * PK + j0, kk);
                if constexpr (KDN) {
                    float uu[8];
                    lds_ld8(U32 + t * PP + j0, uu);
                    const float inv = s_invs[t];
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        w[tt][c] = uu[c] * inv;
                    if (PREP && P.w_out && t < L) {     // gains, for the gradient pass
                        float *wo = P.w_out + (tok0 + (long)t * H) * DK + j0;
                        *reinterpret_cast<float4 *>(wo) =
                            make_float4(w[tt][0], w[tt][1], w[tt][2], w[tt][3]);
                        *reinterpret_cast<float4 *>(wo + 4) =
                            make_float4(w[tt][4], w[tt][5], w[tt][6], w[tt][7]);
                    }
                } else {
                    const float bt = s_beta[t];
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        w[tt][c] = bt * kk[c];
                }
                if constexpr (DECAY) {
                    float qq[8], o[8];
                    lds_ld8(Qt + t * PK + j0, qq);
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        // this token's decay (in registers from the group load)
                        float at = 1.f;
#pragma unroll
                        for (int t2 = 0; t2 < TPG; ++t2)
                            if (ug0 + t2 == t) at = a8[t2][c];
                        ap[tt][c] = at;
                        pre[c] *= at;                   // gamma_t
                    }
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        o[c] = pre[c] * kk[c];
                    lds_st8(Kt + t * PK + j0, o);
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        o[c] = pre[c] * qq[c];
                    lds_st8(Qt + t * PK + j0, o);
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        o[c] = fb ? w[tt][c] : w[tt][c] * fast_rcp(pre[c]);
                    lds_st8(Wp + t * PK + j0, o);
                } else {
                    lds_st8(Wp + t * PK + j0, w[tt]);
                }
            }
            // W~^T[i][t] = (gamma_C / gamma_t) w_t
            float wt[8][TPG2];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                float sg = DECAY ? suf[c] : 1.f;
#pragma unroll
                for (int tt = TPG2 - 1; tt >= 0; --tt) {
                    wt[c][tt] = sg * w[tt][c];
                    if (DECAY)
                        sg *= ap[tt][c];
                }
            }
#pragma unroll
            for (int c = 0; c < 8; ++c)
                lds_stn<TPG2>(WtT + (j0 + c) * PC + u0, wt[c]);
        }
        __syncthreads();

        }
        // ---------------- 3. interaction matrices ----------------
        if constexpr (SPREP) {
            // A_kk = (K K^T) . gamma_t / gamma_s . beta_s (s < t), A_qk likewise
            // with Q (s <= t): raw products from phase 2s, decay applied here
#pragma unroll
            for (int k = 0; k < SPT; ++k) {
                const int x = wv - 1 + k * (NW - 1);
                if (wv == 0 || x >= 2 * NL) continue;
                const int which = x >= NL;
                int idx = x - which * NL, mi = 0;
                while (idx > mi) { idx -= mi + 1; ++mi; }
                const int ni = idx;
                const f32x4 acc = spacc[k];
                const int s = ni * 16 + (lane & 15);
                const float gls = s_gl[s], bs = s_beta[s];
                const int t0r = mi * 16 + (lane >> 4) * 4;
                float val[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {         // branch-free epilogue
                    const int t = t0r + r;
                    const int zt = s_zr[t];
                    const float ex = __builtin_amdgcn_exp2f(fminf(s_gl[t] - gls, 0.f));
                    const bool keep = (which ? s <= t : s < t) & (zt <= s);
                    val[r] = keep ? acc[r] * ex * bs : 0.f;
                }
                if (which) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        AQ[(t0r + r) * PC + s] = from_f32<E>(val[r]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Akk[(t0r + r) * PA + s] = val[r];
                }
            }
        } else if (!fb) {
            for (int x = wv; x < 2 * NL; x += NW) {
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
            stage_rows<E, DK, C, NT>(Kt, PK, gk + tok0 * DK, sk_, L, 0.f, tid);
            stage_rows<E, DK, C, NT>(Qt, PK, gq + tok0 * DK, sk_, L, 0.f, tid);
            __syncthreads();
            for (int pidx = tid; pidx < C * C; pidx += NT) {
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
        for (int x = tid; x < C * C; x += NT) {
            const int t = x / C, s = x % C;
            if ((s >> 4) > (t >> 4)) {
                AQ[t * PC + s] = from_f32<E>(0.f);
                Tm[t * PC + s] = from_f32<E>(0.f);
            }
        }
        __syncthreads();

        // ---------------- 5. U = V - K~ S  ||  4a. T[I,I] ----------------
        constexpr int NTU = NB * NTJ;
        static_assert(NW >= 4 + NB, "waves 0-3 take U, waves 4.. the T blocks");
        if (PREP && wv < 4) {
            // record parts that do not need T, written by waves 0-3 while
            // waves 4.. invert the diagonal blocks
            const WsLayout LW = WsLayout::make(sizeof(E) == 2, C, DK);
            char *rec = static_cast<char *>(P.ws) + ((long)bh * NC + c0 / C) * LW.rec;
            // permuted (chain kernel) records hold -W~^T and -A_qk
            if constexpr (SPREP) {
                const float sg = perm ? -1.f : 1.f;
                store_frag_fn<E, C, DK, 256>(rec + LW.off_kd, tid, perm, [&](int t, int i) {
                    return ld(Kt + t * PK + i) * s_gt[t]; });
                store_frag_fn<E, C, DK, 256>(rec + LW.off_qd, tid, perm, [&](int t, int i) {
                    return ld(Qt + t * PK + i) * s_gt[t]; });
                // W~^T (strided reads of K): half here, half on waves 4-7 below
                store_frag_fn<E, DK, C, 512>(rec + LW.off_wdt, tid, perm, [&](int i, int t) {
                    return ld(Kt + t * PK + i) * (sg * s_wsc[t]); });
            } else {
                store_frag<E, C, DK, 256>(rec + LW.off_kd, Kt, PK, tid, perm);
                store_frag<E, C, DK, 256>(rec + LW.off_qd, Qt, PK, tid, perm);
                store_frag<E, DK, C, 256>(rec + LW.off_wdt, WtT, PC, tid, perm, perm);
            }
            store_frag<E, C, C, 256>(rec + LW.off_aqk, AQ, PC, tid, perm, perm);
        } else if (!PREP && wv < 4) {
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
        } else if (wv >= 4 && wv - 4 < NB) {
            // T[I,I] = (I + A[I,I])^-1, one wave per block, as 2 x 2 blocks of
            // 8 x 8:  T1 = (I + A11)^-1 and T2 = (I + A22)^-1 by forward
            // substitution (lane j < 8: column j of T1, lane 8 + j: column j
            // of T2), then T21 = -T2 A21 T1 on all 64 lanes, one element
            // each.  The block goes to its TD slot (row-major, pitch 20);
            // LDS accesses of one wave complete in order, so the wave reads
            // back what it wrote without a barrier.
            const int I = wv - 4, o0 = I * 16;
            float *td = TD + I * 320;
            if (lane < 16) {
                const int h = lane >> 3, j = lane & 7, off = h * 8;
                const float *arow0 = Akk + (o0 + off) * PA + o0 + off;
                float xv[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const float4 a0 = *reinterpret_cast<const float4 *>(arow0 + r * PA);
                    const float4 a1 = *reinterpret_cast<const float4 *>(arow0 + r * PA + 4);
                    const float ar[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
                    for (int m = 0; m < r; ++m) {
                        if (m & 1) acc1 += ar[m] * xv[m];
                        else acc0 += ar[m] * xv[m];
                    }
                    xv[r] = (r == j) ? 1.f : ((r < j) ? 0.f : -(acc0 + acc1));
                }
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    td[(off + r) * 20 + off + j] = xv[r];
                    if (h == 0)
                        td[r * 20 + 8 + j] = 0.f;          // upper-right block
                }
            }
            __builtin_amdgcn_wave_barrier();
            {
                const int i = lane >> 3, j = lane & 7;      // element (i, j) of the 8 x 8
                const float *a21 = Akk + (o0 + 8 + i) * PA + o0;
                const float4 a0 = *reinterpret_cast<const float4 *>(a21);
                const float4 a1 = *reinterpret_cast<const float4 *>(a21 + 4);
                const float ar[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                float y = 0.f;                              // (A21 T1)[i][j]
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    y += ar[k] * td[k * 20 + j];
                td[i * 20 + 8 + j] = y;                     // parked in the upper right
                __builtin_amdgcn_wave_barrier();
                const float4 t0 = *reinterpret_cast<const float4 *>(td + (8 + i) * 20 + 8);
                const float4 t1 = *reinterpret_cast<const float4 *>(td + (8 + i) * 20 + 12);
                const float t2r[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
                float z = 0.f;                              // (T2 A21 T1)[i][j]
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    z += t2r[k] * td[k * 20 + 8 + j];
                __builtin_amdgcn_wave_barrier();
                td[(8 + i) * 20 + j] = -z;
                td[i * 20 + 8 + j] = 0.f;
            }
            __builtin_amdgcn_wave_barrier();
            {
                // T[I,I] in the operand type, and its transpose (the B operand
                // of the block products); lane: row r, columns c0 .. c0 + 3
                const int r = lane >> 2, c0 = (lane & 3) * 4;
                const float4 t = *reinterpret_cast<const float4 *>(td + r * 20 + c0);
                const float tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Tm[(o0 + r) * PC + o0 + c0 + e] = from_f32<E>(tv[e]);
                if (I < NB - 1) {
                    float *dst = TD + (NB + I) * 320;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dst[(c0 + e) * 20 + r] = tv[e];
                }
            }
        }
        if (SPREP && wv >= 4) {
            // scalar-decay record W~^T[i][t] = beta_t gamma_C / gamma_t k_ti:
            // the other half of its units, after this wave's diagonal block
            const WsLayout LW = WsLayout::make(sizeof(E) == 2, C, DK);
            char *rec = static_cast<char *>(P.ws) + ((long)bh * NC + c0 / C) * LW.rec;
            const float sg = perm ? -1.f : 1.f;     // -W~^T in permuted records
            store_frag_fn<E, DK, C, 512>(rec + LW.off_wdt, tid, perm, [&](int i, int t) {
                return ld(Kt + t * PK + i) * (sg * s_wsc[t]); });
        }
        __syncthreads();
        // ---------------- 4b. off-diagonal blocks of T ----------------
        if constexpr (PREP) {
            // With D = diag(T[I,I]) and N the blocks of A below the diagonal,
            // I + A = (I + N D) D^-1, so T = D X with X = (I + M)^-1, M = N D:
            //   M[I,K] = A[I,K] T[K,K];  X[I,I-1] = -M[I,I-1],
            //   X[2,0] = -M[2,0] + M[2,1] M[1,0],  X[3,1] = -M[3,1] + M[3,2] M[2,1],
            //   X[3,0] = -M[3,0] + M[3,1] M[1,0] - M[3,2] X[2,0];  T[I,K] = T[I,I] X[I,K].
            // Three levels of independent 16 x 16 products on waves 0-5 (four
            // products deep) instead of one chain per column.  Scratch: 16 x 20
            // slots over K~ / Q~, free once their records are written.  "t"
            // slots hold the transpose (the B operand of mma16_f32), row slots
            // the matrix (its A operand).
            static_assert(LY::OFF_QT == LY::OFF_KT + LY::SZ_CK &&
                              (NB == 2 ? 1 : 12) * 320 * 4 <= 2 * LY::SZ_CK,
                          "scratch slots fit over K~ and Q~");
            float *SL = reinterpret_cast<float *>(smem + LY::OFF_KT);
            auto slot = [&](int n) { return SL + n * 320; };
            auto tdiag = [&](int I) { return TD + I * 320; };            // T[I,I]
            auto tdiag_t = [&](int I) { return TD + (NB + I) * 320; };   // T[I,I]^T
            auto akk = [&](int I, int K) { return Akk + I * 16 * PA + K * 16; };
            const int col = lane & 15, row0 = (lane >> 4) * 4;
            auto put_t = [&](float *d, const f32x4 &v) {
                *reinterpret_cast<float4 *>(d + col * 20 + row0) = make_float4(v[0], v[1], v[2], v[3]);
            };
            auto put_row = [&](float *d, const f32x4 &v) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    d[(row0 + r) * 20 + col] = v[r];
            };
            auto get_t = [&](const float *d) {
                const float4 x = *reinterpret_cast<const float4 *>(d + col * 20 + row0);
                return f32x4{x.x, x.y, x.z, x.w};
            };
            // T[I,K] = sgn T[I,I] X (X^T in xt) into Tm
            auto put_tm = [&](int I, int K, const float *xt, float sgn) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                mma16_f32<E>(acc, tdiag(I), 20, xt, 20, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Tm[(I * 16 + row0 + r) * PC + K * 16 + col] = from_f32<E>(sgn * acc[r]);
            };
            if constexpr (NB == 2) {
                if (wv == 0) {                 // T[1,0] = -T[1,1] A[1,0] T[0,0]
                    f32x4 m = {0.f, 0.f, 0.f, 0.f};
                    mma16_f32<E>(m, akk(1, 0), PA, tdiag_t(0), 20, lane);
                    put_t(slot(0), m);
                    put_tm(1, 0, slot(0), -1.f);
                }
            } else {
                static_assert(NB == 4, "chunk of 32 or 64");
                // slots: M10t 0, M21 1 (row) 2 (t), M32 3 (row) 4 (t), M20t 5,
                //        M31 6 (row) 7 (t), M30t 8, X20t 9, X31t 10, Y30t 11, X30t 5
                constexpr int LI[6] = {1, 2, 3, 2, 3, 3}, LK[6] = {0, 1, 2, 0, 1, 0};
                if (wv < 6) {                  // level 1: M = A[I,K] T[K,K]
                    const int I = LI[wv], K = LK[wv];
                    f32x4 m = {0.f, 0.f, 0.f, 0.f};
                    mma16_f32<E>(m, akk(I, K), PA, tdiag_t(K), 20, lane);
                    if (wv == 0) put_t(slot(0), m);
                    if (wv == 1) { put_row(slot(1), m); put_t(slot(2), m); }
                    if (wv == 2) { put_row(slot(3), m); put_t(slot(4), m); }
                    if (wv == 3) put_t(slot(5), m);
                    if (wv == 4) { put_row(slot(6), m); put_t(slot(7), m); }
                    if (wv == 5) put_t(slot(8), m);
                }
                __syncthreads();
                if (wv < 3) {                  // level 2: T[I,I-1] = -T[I,I] M[I,I-1]
                    const int I = wv + 1;
                    put_tm(I, I - 1, slot(wv == 0 ? 0 : (wv == 1 ? 2 : 4)), -1.f);
                } else if (wv < 6) {           // X[2,0], X[3,1], Y = -M[3,0] + M[3,1] M[1,0]
                    const int ia = wv == 3 ? 1 : (wv == 4 ? 3 : 6);   // A operand (row)
                    const int ib = wv == 3 ? 0 : (wv == 4 ? 2 : 0);   // B operand (t)
                    const int ic = wv == 3 ? 5 : (wv == 4 ? 7 : 8);   // -initial (t)
                    f32x4 acc = get_t(slot(ic));
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[r] = -acc[r];
                    mma16_f32<E>(acc, slot(ia), 20, slot(ib), 20, lane);
                    put_t(slot(6 + wv), acc);                         // X20t 9, X31t 10, Y30t 11
                }
                __syncthreads();
                if (wv == 0) {
                    put_tm(2, 0, slot(9), 1.f);                       // T[2,0] = T[2,2] X[2,0]
                } else if (wv == 1) {
                    put_tm(3, 1, slot(10), 1.f);                      // T[3,1] = T[3,3] X[3,1]
                } else if (wv == 2) {                                 // X[3,0] = Y - M[3,2] X[2,0]
                    f32x4 p = {0.f, 0.f, 0.f, 0.f};
                    mma16_f32<E>(p, slot(3), 20, slot(9), 20, lane);
                    f32x4 x = get_t(slot(11));
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        x[r] -= p[r];
                    put_t(slot(5), x);          // read back by this wave only
                    put_tm(3, 0, slot(5), 1.f);
                }
            }
            __syncthreads();
        } else {
            // Column chain J on wave J (no barriers between its steps):
            //   T[I,J] = -T[I,I] sum_{K=J}^{I-1} A[I,K] T[K,J],  I = J+1 .. NB-1.
            // Products in (near) fp32: bf16 data is split into hi + lo parts.
            if (wv < NB - 1) {
                const int J = wv;
                // private slots of wave J: P^T, then T[K,J]^T for K = J+1 .. NB-2
                float *ps = TD + (NB + (NB - 1) + J * (2 * NB - 1 - J) / 2) * 320;
                for (int I = J + 1; I < NB; ++I) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    for (int K = J; K < I; ++K) {
                        const float *bk = (K == J) ? TD + (NB + J) * 320 : ps + (K - J) * 320;
                        mma16_f32<E>(acc, Akk + I * 16 * PA + K * 16, PA, bk, 20, lane);
                    }
                    *reinterpret_cast<float4 *>(ps + (lane & 15) * 20 + (lane >> 4) * 4) =
                        make_float4(acc[0], acc[1], acc[2], acc[3]);
                    f32x4 tij = {0.f, 0.f, 0.f, 0.f};
                    mma16_f32<E>(tij, TD + I * 320, 20, ps, 20, lane);
                    const int col = J * 16 + (lane & 15), row0 = I * 16 + (lane >> 4) * 4;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Tm[(row0 + r) * PC + col] = from_f32<E>(-tij[r]);
                    if (I < NB - 1)                    // T[I,J]^T for later steps
                        *reinterpret_cast<float4 *>(ps + (I - J) * 320 + (lane & 15) * 20 +
                                                    (lane >> 4) * 4) =
                            make_float4(-tij[0], -tij[1], -tij[2], -tij[3]);
                }
            }
            __syncthreads();
        }
        if constexpr (PREP) {
            // ---------------- record of this chunk ----------------
            const WsLayout LW = WsLayout::make(sizeof(E) == 2, C, DK);
            char *rec = static_cast<char *>(P.ws) + ((long)bh * NC + c0 / C) * LW.rec;
            store_frag<E, C, C, NT>(rec + LW.off_tm, Tm, PC, tid, perm);
            if (DECAY && tid < DK)
                reinterpret_cast<float *>(rec + LW.off_gc)[tid] = s_gc[tid];
            __syncthreads();            // LDS reads done before the next commit
            continue;
        }

        // ---------------- 6. E = T U ----------------
        for (int x = wv; x < NTU; x += NW) {
            const int mi = x / NTJ, nj = x % NTJ;
            const int kc = min(C, ((mi + 1) * 16 + KS - 1) / KS * KS);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile<E>(acc, Tm + mi * 16 * PC, PC, UT + nj * 16 * PC, PC, kc, lane);
            const int j = nj * 16 + (lane & 15);
            float eo[4] = {acc[0], acc[1], acc[2], acc[3]};
            lds_stn<4>(ET + j * PC + mi * 16 + (lane >> 4) * 4, eo);
        }
        __syncthreads();

        // ---------------- 7. outputs and state ----------------
        E *go = static_cast<E *>(P.o);
        for (int x = wv; x < NTU; x += NW) {
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
            const int tau = wv + NW * u, ti = tau / NTJ, tj = tau % NTJ;
        if (NST % NW != 0 && tau >= NST) continue;
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
            const int tau = wv + NW * u, ti = tau / NTJ, tj = tau % NTJ;
        if (NST % NW != 0 && tau >= NST) continue;
            const int j = tj * 16 + (lane & 15);
            float so[4] = {sacc[u][0], sacc[u][1], sacc[u][2], sacc[u][3]};
            lds_stn<4>(ST + j * PK + ti * 16 + (lane >> 4) * 4, so);
        }
    }

    // ---- final state
    if constexpr (PREP)
        return;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int tau = wv + NW * u, ti = tau / NTJ, tj = tau % NTJ;
        if (NST % NW != 0 && tau >= NST) continue;
        const int j = tj * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ti * 16 + (lane >> 4) * 4 + r;
            P.S_out[((long)bh * DK + i) * DV + v0 + j] = sacc[u][r];
        }
    }
    if (KDN && vb == 0 && tid < DK)
        P.p_out[(long)bh * DK + tid] = p_reg;
    if (ISO && vb == 0 && tid == 0)
        P.p_out[bh] = p_reg;
}
#endif  // KDN_PREFILL_VARIANT

// ---------------------------------------------------------------------------
// Host-side dispatch.  This file is compiled once per variant
// (KDN_PREFILL_VARIANT = 0..4, each unit instantiates that variant's kernels)
// and once with KDN_PREFILL_DISPATCH for the entry point below.
// ---------------------------------------------------------------------------
#ifdef KDN_PREFILL_VARIANT
#ifndef KDN_PREFILL_WAVES
#define KDN_PREFILL_WAVES 8
#endif
template <typename E, int VAR, int DK, int NV, int C>
static hipError_t launch_one(const PrefillParams &P, hipStream_t st) {
    constexpr int NW = KDN_PREFILL_WAVES;
    const long heads = (long)P.B * P.H;
    const dim3 grid((unsigned)(heads * (P.dv / NV))), block(64 * NW);
    hipLaunchKernelGGL((prefill_kernel<E, VAR, DK, NV, C, NW, false>), grid, block, 0, st, P);
    return hipGetLastError();
}

template <typename E, int VAR, int DK, int C>
static hipError_t launch_prep_one(const PrefillParams &P, hipStream_t st) {
    constexpr int NW = KDN_PREFILL_WAVES;
    const long units = (long)P.B * P.H * ((P.T + C - 1) / C);
    // persistent: one workgroup per CU (the LDS footprint allows one), each
    // walking every gridDim-th (batch*head, chunk) unit
    const long g = units < P.cus ? units : P.cus;
    const dim3 grid((unsigned)g), block(64 * NW);
    hipLaunchKernelGGL((prefill_kernel<E, VAR, DK, 16, C, NW, true>), grid, block, 0, st, P);
    return hipGetLastError();
}

template <typename E, int VAR>
static hipError_t launch_prep_var(const PrefillParams &P, hipStream_t st) {
    if (P.dk == 128 && P.chunk == 64) {
        if constexpr (sizeof(E) == 2)
            return launch_prep_one<E, VAR, 128, 64>(P, st);
        return hipErrorInvalidValue;
    }
    if (P.dk == 128 && P.chunk == 32) return launch_prep_one<E, VAR, 128, 32>(P, st);
    if (P.dk == 64 && P.chunk == 64) return launch_prep_one<E, VAR, 64, 64>(P, st);
    if (P.dk == 64 && P.chunk == 32) return launch_prep_one<E, VAR, 64, 32>(P, st);
    return hipErrorInvalidValue;
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
hipError_t KDN_CAT(launch_prefill_prep_v, KDN_PREFILL_VARIANT)(const PrefillParams &P,
                                                               hipStream_t st) {
    return P.bf16 ? launch_prep_var<bf16, KDN_PREFILL_VARIANT>(P, st)
                  : launch_prep_var<float, KDN_PREFILL_VARIANT>(P, st);
}
#endif  // KDN_PREFILL_VARIANT

#ifdef KDN_PREFILL_DISPATCH
int prefill_value_block(const PrefillParams &P) {
    // Enough workgroups to cover the device's CUs, value blocks of 16 or 32
    // columns (float32 operands: 16, for the LDS budget).
    if (!P.bf16)
        return 16;
    const long heads = (long)P.B * P.H;
    int nv = 32;
    while (nv > 16 && heads * (P.dv / nv) < P.cus)
        nv >>= 1;
    return nv;
}

long long prefill_workspace_bytes(int variant, int bf16, long long B, long long T,
                                  long long H, int dk, int C) {
    const long long bh = B * H, nc = num_chunks(T, C);
    long long n = WsLayout::make(bf16, C, dk).records(bh, nc);
    if (variant == DIAG_KDN)
        n += WsLayout::mobius_bytes(bh, nc, dk) + WsLayout::p0_bytes(bh, nc, dk) +
             WsLayout::pre_bytes(bh, nc, dk);
    if (variant == ISO_KDN)
        n += WsLayout::mobius_bytes(bh, nc, 1) + WsLayout::stat_bytes(bh, nc, C) +
             WsLayout::p0_bytes(bh, nc, 1);
    return n;
}

static hipError_t launch_two_pass(const PrefillParams &P, hipStream_t st) {
    hipError_t e = hipSuccess;
    if ((P.variant == DIAG_KDN || P.variant == ISO_KDN) &&
        (e = launch_variance_scan(P, st)) != hipSuccess)
        return e;
    if (P.T > 0) {
        switch (P.variant) {
        case DELTANET: e = launch_prefill_prep_v0(P, st); break;
        case GATED_DELTANET: e = launch_prefill_prep_v1(P, st); break;
        case KDA: e = launch_prefill_prep_v2(P, st); break;
        case DIAG_KDN: e = launch_prefill_prep_v3(P, st); break;
        case ISO_KDN: e = launch_prefill_prep_v4(P, st); break;
        default: e = hipErrorInvalidValue;
        }
        if (e != hipSuccess)
            return e;
    }
    return P.rec_perm ? launch_prefill_chain(P, st) : launch_prefill_state(P, st);
}

hipError_t launch_prefill(const PrefillParams &P, hipStream_t st) {
    if ((long)P.B * P.H == 0)
        return hipSuccess;
    // a few tokens per sequence (e.g. draft tokens checked against a resident
    // state): one workgroup per head, whatever the schedule asked for
    if (P.bf16 && P.T > 0 && P.T <= PREFILL_SHORT_T)
        return launch_prefill_short(P, st);
    if (P.ws)
        return launch_two_pass(P, st);
    const int nv = prefill_value_block(P);
    switch (P.variant) {
    case DELTANET: return launch_prefill_v0(P, st, nv);
    case GATED_DELTANET: return launch_prefill_v1(P, st, nv);
    case KDA: return launch_prefill_v2(P, st, nv);
    case DIAG_KDN: return launch_prefill_v3(P, st, nv);
    case ISO_KDN: return launch_prefill_v4(P, st, nv);
    }
    return hipErrorInvalidValue;
}
#endif  // KDN_PREFILL_DISPATCH

}  // namespace kdn
