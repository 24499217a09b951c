// kdn_backward.hip -- gradients of the chunkwise prefill (gfx950): the
// memory part of every variant (DeltaNet, Gated DeltaNet, KDA; the KDN
// variants through KDA's with their derived write vectors) and the adjoints
// of the KDN variance chains.
//
// The forward chunk algebra (page "معماری KDA: حذف تداخل حافظه با قانون دلتا در
// توالی‌های بلند", section "حل مشکل وابستگی علی"), per chunk entering with state S:
//   U = V - K~ S,  E = T U,  O = Q~ S + A_qk E,  S' = diag(gamma_C) S + W~^T E,
// with T = (I + A_kk)^-1.  Its exact reverse, for cotangents dO of the outputs
// and dS' of the state leaving the chunk:
//   dE = A_qk^T dO + W~ dS',   dU = T^T dE,   dV = dU,
//   dS = diag(gamma_C) dS' + Q~^T dO - K~^T dU                    (state pass)
//   dA_qk = tril(dO E^T),  dA_kk = strict tril(-dU E^T)          (local)
//   dQ~ = dO S^T + dA_qk W',  dK~ = -dU S^T + dA_kk W',
//   dW' = dA_qk^T Q~ + dA_kk^T K~ + diag(gamma_C) E dS'^T,
// where A_kk = K~ W'^T, A_qk = Q~ W'^T, W' = w / gamma, W~ = gamma_C W'.  Back
// through the decay scaling (K~ = gamma k, Q~ = gamma q, w = beta k):
//   dq = gamma dQ~,  dw = dW' / gamma,  dk = gamma dK~ + beta dw,  dbeta = k . dw,
//   d log gamma_t = k (gamma dK~) + q dq - w dw  (+ the gamma_C terms at the
//   chunk end), and d log a_r = sum over t >= r of d log gamma_t.
//
// Two launches after the forward pass (which saves S at every chunk start):
//   backward_state_kernel: one workgroup per (batch*head, value block) walks
//     the chunks in reverse, dS in registers, and saves dS' of every chunk;
//   backward_chunk_kernel: one workgroup per (batch*head, chunk) forms the
//     chunk's local gradients from S, dS', the tiles and the forward record.
// For KDN three more reverse the variance chain (map, scan over chunks,
// per-token gradients).
#include "kdn_device.h"
#include "kdn_launch.h"
#include "kdn_workspace.h"

namespace kdn {

#ifdef KDN_DECAY_FLOOR
#undef KDN_DECAY_FLOOR
#endif
// Below this cumulative in-chunk decay the 1/gamma operand scaling is not
// used; the chunk takes the exact elementwise path.
#define KDN_DECAY_FLOOR 8.077935669463161e-28f   /* 2^-90 */

// The 16-byte units of a record matrix X[R][K] (fragment order,
// kdn_workspace.h) that thread tid moves: units tid + NT n.  load() issues all
// of them before any is used; store() writes X to LDS as dst[r * pitch + k]
// or, TRANS, as X^T: dst[k * pitch + r] (times sgn).
template <typename E, int R, int K, int NT>
struct RecUnits {
    static constexpr int EPU = 16 / (int)sizeof(E);
    static constexpr int KG = sizeof(E) == 2 ? 32 : 16;
    static constexpr int NU = R * K / EPU;
    static constexpr int NPT = (NU + NT - 1) / NT;
    uint4 u[NPT];
    __device__ __forceinline__ void load(const char *src, int tid) {
        const uint4 *s = reinterpret_cast<const uint4 *>(src);
#pragma unroll
        for (int n = 0; n < NPT; ++n) {
            const int x = tid + NT * n;
            if (NU % NT == 0 || x < NU)
                u[n] = s[x];
        }
    }
    // perm (bf16): the record's contraction index is in the permuted order
    // of the chain kernel's records (each 32-group: a lane's 8 elements are
    // columns 4q..4q+3 and 16+4q..16+4q+3), restored here
    template <bool TRANS>
    __device__ __forceinline__ void store(E *dst, int pitch, float sgn, int tid,
                                          bool perm) const {
#pragma unroll
        for (int n = 0; n < NPT; ++n) {
            const int x = tid + NT * n;
            if (!(NU % NT == 0 || x < NU)) continue;
            const int l = x & 63, grp = x >> 6;
            const int m = grp / (K / KG), g = grp % (K / KG);
            const int row = m * 16 + (l & 15);
            if (!TRANS && sizeof(E) == 2 && sgn == 1.f) {
                if (perm) {
                    E *d = dst + row * pitch + g * 32 + (l >> 4) * 4;
                    *reinterpret_cast<uint2 *>(d) = make_uint2(u[n].x, u[n].y);
                    *reinterpret_cast<uint2 *>(d + 16) = make_uint2(u[n].z, u[n].w);
                } else {
                    *reinterpret_cast<uint4 *>(dst + row * pitch + g * 32 + (l >> 4) * 8) = u[n];
                }
                continue;
            }
            if (TRANS && sizeof(E) == 2) {
                // Lanes l and l^1 hold rows r and r+1 (r even) of the same 8
                // columns: they swap halves (one DPP quad permute per dword),
                // then each writes 4 dwords, rows (r, r+1) of one column each
                // (the even lane columns 0-3, the odd lane columns 4-7).
                const bool odd = l & 1;
                const uint32_t flip = sgn < 0.f ? 0x80008000u : 0u;   // exact bf16 negation
                const uint32_t w0 = u[n].x ^ flip, w1 = u[n].y ^ flip;
                const uint32_t w2 = u[n].z ^ flip, w3 = u[n].w ^ flip;
                const uint32_t m0 = odd ? w2 : w0, m1 = odd ? w3 : w1;   // kept
                const uint32_t s0 = odd ? w0 : w2, s1 = odd ? w1 : w3;   // sent
                const uint32_t r0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s0, 0xB1, 0xf, 0xf, false);
                const uint32_t r1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s1, 0xB1, 0xf, 0xf, false);
                const uint32_t lo0 = odd ? r0 : m0, lo1 = odd ? r1 : m1;   // row r
                const uint32_t hi0 = odd ? m0 : r0, hi1 = odd ? m1 : r1;   // row r + 1
                const int col = perm ? g * 32 + (l >> 4) * 4 + (odd ? 16 : 0)
                                     : g * 32 + (l >> 4) * 8 + (odd ? 4 : 0);
                uint32_t *d = reinterpret_cast<uint32_t *>(dst + col * pitch + (row & ~1));
                const int pw = pitch / 2;                                  // dwords per row
                d[0] = (lo0 & 0xffffu) | (hi0 << 16);
                d[pw] = (lo0 >> 16) | (hi0 & 0xffff0000u);
                d[2 * pw] = (lo1 & 0xffffu) | (hi1 << 16);
                d[3 * pw] = (lo1 >> 16) | (hi1 & 0xffff0000u);
                continue;
            }
            const uint4 v = u[n];
            const E *e = reinterpret_cast<const E *>(&v);
#pragma unroll
            for (int xx = 0; xx < EPU; ++xx) {
                const int col = sizeof(E) == 2
                                    ? (perm ? g * 32 + (l >> 4) * 4 + (xx < 4 ? xx : 12 + xx)
                                            : g * 32 + (l >> 4) * 8 + xx)
                                    : g * 16 + xx * 4 + (l >> 4);
                const E val = from_f32<E>(sgn * to_f32(e[xx]));
                if (TRANS)
                    dst[col * pitch + row] = val;
                else
                    dst[row * pitch + col] = val;
            }
        }
    }
};

// Four consecutive elements of E from global memory, held raw (as loaded)
// and converted where used, so no wait follows the load.
template <typename E> struct Raw4;
template <> struct Raw4<float> {
    float4 v;
    __device__ __forceinline__ void load(const float *p) { v = *reinterpret_cast<const float4 *>(p); }
    __device__ __forceinline__ void store(float *p) const { *reinterpret_cast<float4 *>(p) = v; }
    __device__ __forceinline__ float operator[](int e) const {
        return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    }
};
template <> struct Raw4<bf16> {
    uint2 v;
    __device__ __forceinline__ void load(const bf16 *p) { v = *reinterpret_cast<const uint2 *>(p); }
    __device__ __forceinline__ void store(bf16 *p) const { *reinterpret_cast<uint2 *>(p) = v; }
    __device__ __forceinline__ float operator[](int e) const {
        const uint32_t w = e < 2 ? v.x : v.y;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

// Four consecutive elements of E from global memory as floats.
__device__ __forceinline__ void gload4(const float *p, float (&f)[4]) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}
__device__ __forceinline__ void gload4(const bf16 *p, float (&f)[4]) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
}

// ---------------------------------------------------------------------------
// Reverse state pass.  Per chunk, from the chunk's record:
//   dE = A_qk^T dO + W~ dS,  dU = T^T dE,  dS <- diag(gamma_C) dS + Q~^T dO - K~^T dU.
// LDS operands (row = MFMA row, k contiguous): A_qk^T [s][t], W~ [s][i],
// T^T [t][s], Q~^T [i][t], -K~^T [i][t]; the B operands dO^T, dS^T, dE^T,
// dU^T as [column][k].
// ---------------------------------------------------------------------------
template <typename E, bool DECAY, int DK, int NV, int C>
__global__ __launch_bounds__(512) void backward_state_kernel(BackwardParams P) {
    constexpr int NT = 512, NW = 8;
    constexpr int PADE = 16 / (int)sizeof(E);
    constexpr int PK = DK + PADE, PC = C + PADE;
    constexpr int NTJ = NV / 16, NTI = DK / 16, NTC = C / 16;
    constexpr int NSS = (NTI * NTJ + NW - 1) / NW;   // dS tiles per wave
    constexpr int NSE = (NTC * NTJ + NW - 1) / NW;   // dE / dU tiles per wave

    __shared__ __attribute__((aligned(16))) E AQT[C * PC];
    __shared__ __attribute__((aligned(16))) E WR[C * PK];
    __shared__ __attribute__((aligned(16))) E TT[C * PC];
    __shared__ __attribute__((aligned(16))) E QT[DK * PC];
    __shared__ __attribute__((aligned(16))) E KT[DK * PC];
    __shared__ __attribute__((aligned(16))) E DOT[NV * PC];
    __shared__ __attribute__((aligned(16))) E DST[NV * PK];
    __shared__ __attribute__((aligned(16))) E DET[NV * PC];
    __shared__ __attribute__((aligned(16))) E DUT[NV * PC];
    __shared__ float GC[DK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // records in the chain kernel's permuted column order (bf16 calls)
    const bool perm = sizeof(E) == 2 && P.rec_perm != 0;
    // Workgroup -> (batch*head, value block).  Dispatch is round-robin over
    // the 8 XCDs; the value blocks of one head go to one XCD, so each chunk's
    // record crosses HBM once and the other blocks read it from that L2.
    const int nvb = P.dv / NV;
    const int G = gridDim.x;
    int lid = blockIdx.x;
    if ((G & 7) == 0 && ((G >> 3) % nvb) == 0)
        lid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int bh = lid / nvb, vb = lid % nvb;
    const int b = bh / P.H, h = bh % P.H;
    const int v0 = vb * NV;
    const int T = P.T, H = P.H, DV = P.dv;
    const int NC = (T + C - 1) / C;
    const WsLayout LW = WsLayout::make(sizeof(E) == 2, C, DK);
    const char *ws = static_cast<const char *>(P.ws) + (long)bh * NC * LW.rec;
    const E *gdo = static_cast<const E *>(P.dO);

    // dS tiles: tau = wv + NW k -> (key tile, column tile) = (tau / NTJ, tau % NTJ)
    f32x4 dacc[NSS];
#pragma unroll
    for (int k = 0; k < NSS; ++k) {
        const int tau = wv + NW * k;
        if (NSS * NW != NTI * NTJ && tau >= NTI * NTJ) continue;
        const int i0 = (tau / NTJ) * 16 + (lane >> 4) * 4, j = (tau % NTJ) * 16 + (lane & 15);
        float s4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dacc[k][r] = P.dS_out ? P.dS_out[((long)bh * DK + i0 + r) * DV + v0 + j] : 0.f;
            s4[r] = dacc[k][r];
        }
        lds_stn<4>(DST + j * PK + i0, s4);
    }

    // One chunk's record units and dO elements, loaded one chunk ahead.
    constexpr int NDO = (C * NV + NT - 1) / NT;
    struct Rec {
        RecUnits<E, C, C, NT> aq, tm;
        RecUnits<E, DK, C, NT> wt;
        RecUnits<E, C, DK, NT> qd, kd;
        float gc;
        E dov[NDO];
    };
    auto load = [&](Rec &X, int c) {
        const char *rec = ws + (long)c * LW.rec;
        X.aq.load(rec + LW.off_aqk, tid);
        X.wt.load(rec + LW.off_wdt, tid);
        X.tm.load(rec + LW.off_tm, tid);
        X.qd.load(rec + LW.off_qd, tid);
        X.kd.load(rec + LW.off_kd, tid);
        // every load unconditional (rows clamped into the sequence, zeroed
        // where used), so all of them are in flight together
        X.gc = DECAY ? reinterpret_cast<const float *>(rec + LW.off_gc)[tid % DK] : 1.f;
        const int L = min(C, T - c * C);
#pragma unroll
        for (int n = 0; n < NDO; ++n) {
            const int x = tid + NT * n, t = min(x / NV, L - 1), j = x % NV;
            const long row = ((long)b * T + c * C + t) * H + h;
            X.dov[n] = gdo[row * DV + v0 + j];
        }
    };
    Rec X;
    if (NC > 0)
        load(X, NC - 1);

    for (int c = NC - 1; c >= 0; --c) {
        // dS leaving this chunk, for the local-gradient kernel
        E *sv = static_cast<E *>(P.dstates) + ((long)bh * NC + c) * DK * DV;
#pragma unroll
        for (int k = 0; k < NSS; ++k) {
            const int tau = wv + NW * k;
            if (NSS * NW != NTI * NTJ && tau >= NTI * NTJ) continue;
            const int i0 = (tau / NTJ) * 16 + (lane >> 4) * 4, j = (tau % NTJ) * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sv[(long)(i0 + r) * DV + v0 + j] = from_f32<E>(dacc[k][r]);
        }
        // permuted (bf16 chain kernel) records hold -A_qk and -W~^T
        X.aq.template store<true>(AQT, PC, perm ? -1.f : 1.f, tid, perm);
        X.wt.template store<true>(WR, PK, perm ? -1.f : 1.f, tid, perm);
        X.tm.template store<true>(TT, PC, 1.f, tid, perm);
        X.qd.template store<true>(QT, PC, 1.f, tid, perm);
        X.kd.template store<true>(KT, PC, -1.f, tid, perm);
        if (DECAY && tid < DK)
            GC[tid] = X.gc;
        const int L = min(C, T - c * C);
#pragma unroll
        for (int n = 0; n < NDO; ++n) {                // dO^T (rows past the end are 0)
            const int x = tid + NT * n;
            if ((C * NV) % NT == 0 || x < C * NV)
                DOT[(x % NV) * PC + x / NV] = x / NV < L ? X.dov[n] : from_f32<E>(0.f);
        }
        if (c > 0)
            load(X, c - 1);                            // in flight during this chunk
        __syncthreads();
        // dE = A_qk^T dO + W~ dS  -> dE^T
#pragma unroll
        for (int k = 0; k < NSE; ++k) {
            const int tau = wv + NW * k;
            if (NSE * NW != NTC * NTJ && tau >= NTC * NTJ) continue;
            const int ms = tau / NTJ, nj = tau % NTJ;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile_k<E, C>(acc, AQT + ms * 16 * PC, PC, DOT + nj * 16 * PC, PC, lane);
            mma_tile_k<E, DK>(acc, WR + ms * 16 * PK, PK, DST + nj * 16 * PK, PK, lane);
            float e4[4] = {acc[0], acc[1], acc[2], acc[3]};
            lds_stn<4>(DET + (nj * 16 + (lane & 15)) * PC + ms * 16 + (lane >> 4) * 4, e4);
        }
        __syncthreads();
        // dU = T^T dE  -> dU^T
#pragma unroll
        for (int k = 0; k < NSE; ++k) {
            const int tau = wv + NW * k;
            if (NSE * NW != NTC * NTJ && tau >= NTC * NTJ) continue;
            const int mt = tau / NTJ, nj = tau % NTJ;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile_k<E, C>(acc, TT + mt * 16 * PC, PC, DET + nj * 16 * PC, PC, lane);
            float u4[4] = {acc[0], acc[1], acc[2], acc[3]};
            lds_stn<4>(DUT + (nj * 16 + (lane & 15)) * PC + mt * 16 + (lane >> 4) * 4, u4);
        }
        __syncthreads();
        // dS <- diag(gamma_C) dS + Q~^T dO - K~^T dU
#pragma unroll
        for (int k = 0; k < NSS; ++k) {
            const int tau = wv + NW * k;
            if (NSS * NW != NTI * NTJ && tau >= NTI * NTJ) continue;
            const int mi = tau / NTJ, nj = tau % NTJ;
            const int i0 = mi * 16 + (lane >> 4) * 4, j = nj * 16 + (lane & 15);
            if (DECAY) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dacc[k][r] *= GC[i0 + r];
            }
            mma_tile_k<E, C>(dacc[k], QT + mi * 16 * PC, PC, DOT + nj * 16 * PC, PC, lane);
            mma_tile_k<E, C>(dacc[k], KT + mi * 16 * PC, PC, DUT + nj * 16 * PC, PC, lane);
            float s4[4] = {dacc[k][0], dacc[k][1], dacc[k][2], dacc[k][3]};
            lds_stn<4>(DST + j * PK + i0, s4);
        }
        __syncthreads();
    }
    if (P.dS0) {
#pragma unroll
        for (int k = 0; k < NSS; ++k) {
            const int tau = wv + NW * k;
            if (NSS * NW != NTI * NTJ && tau >= NTI * NTJ) continue;
            const int i0 = (tau / NTJ) * 16 + (lane >> 4) * 4, j = (tau % NTJ) * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                P.dS0[((long)bh * DK + i0 + r) * DV + v0 + j] = dacc[k][r];
        }
    }
}

// ---------------------------------------------------------------------------
// Local gradients of one chunk.  The value columns are taken in halves of DVH;
// per half (j: the half's columns)
//   U = V - K~ S,  E = T U,  dE = A_qk^T dO + W~ dS',  dU = T^T dE  (dv = dU)
// and the products summed over j go to registers:
//   dQ~ += dO S^T,  dK~ -= dU S^T,  dW~ += E dS'^T,  dA_qk += dO E^T,
//   dA_kk -= dU E^T,  and sum_j S dS' per key channel.
// Then the decay-scaled products dQ~ += dA_qk W', dK~ += dA_kk W',
// dW' = gamma_C dW~ + dA_kk^T K~ + dA_qk^T Q~ (exact elementwise sums over the
// decay ratios when a channel's in-chunk decay drops below 2^-90), and the
// elementwise step to dq, dk, dbeta and d log gamma; finally the reverse sum
// over the chunk's tokens gives d log alpha.
// ---------------------------------------------------------------------------
template <typename E, int DK, int C, int DVH>
struct BwdLayout {
    static constexpr int ES = (int)sizeof(E), PADE = 16 / ES;
    static constexpr int PK = DK + PADE, PC = C + PADE, PH = DVH + PADE, PF = DK + 4;
    static constexpr int SZ_CK = C * PK * ES, SZ_CC = C * PC * ES, SZ_KC = DK * PC * ES;
    static constexpr int SZ_HC = DVH * PC * ES, SZ_CH = C * PH * ES, SZ_KH = DK * PH * ES;
    static constexpr int SZ_SB1 = (DVH * PK > DK * PH ? DVH * PK : DK * PH) * ES;
    static constexpr int SZ_F = C * PF * 4;
    static constexpr int OFF_WR = 0;
    static constexpr int BASE = SZ_CK;
    // chunk and half phases
    static constexpr int OFF_KR = BASE, OFF_TR = OFF_KR + SZ_CK, OFF_TT = OFF_TR + SZ_CC,
                         OFF_AQT = OFF_TT + SZ_CC, OFF_SB1 = OFF_AQT + SZ_CC,
                         OFF_SB2 = OFF_SB1 + SZ_SB1, OFF_UE = OFF_SB2 + SZ_KH,
                         OFF_EH = OFF_UE + SZ_HC, OFF_DOT = OFF_EH + SZ_CH,
                         OFF_DOH = OFF_DOT + SZ_HC, OFF_DUH = OFF_DOH + SZ_CH,
                         END_A = OFF_DUH + SZ_CH;
    // decay-scaled products and the elementwise step (over the same bytes)
    static constexpr int OFF_DAQ = BASE, OFF_DAQT = OFF_DAQ + SZ_CC, OFF_DAK = OFF_DAQT + SZ_CC,
                         OFF_DAKT = OFF_DAK + SZ_CC, OFF_WPT = OFF_DAKT + SZ_CC,
                         OFF_QTT = OFF_WPT + SZ_KC, OFF_KTT = OFF_QTT + SZ_KC,
                         OFF_GAM = OFF_KTT + SZ_KC, END_F = OFF_GAM + SZ_F;
    static constexpr int OFF_DG = BASE;   // over the dA matrices and W'^T, Q~^T, K~^T
    static constexpr int END = END_A > END_F ? END_A : END_F;
    static constexpr int OFF_SM = END;
    static constexpr int SM_GC = 0, SM_DGC = DK, SM_SDS = 2 * DK, SM_DB = 3 * DK,
                         SM_DLA = 3 * DK + C, SM_FLAG = 3 * DK + 2 * C;
    static constexpr int TOTAL = OFF_SM + (3 * DK + 2 * C + 4) * 4;
    static_assert(OFF_DG + SZ_F <= OFF_GAM, "d log gamma clear of gamma");
    static_assert(TOTAL <= 163840, "backward LDS budget");
};

// Source of the write vector w of each token: beta k with beta given (the
// write-strength variants), beta k with beta derived by the forward pass
// (isotropic KDN, float32), or the gain saved by the forward pass (diagonal
// KDN).  A template argument, so every load of the kernel is unconditional.
enum WriteSrc { WS_BETA = 0, WS_BETA_F32 = 1, WS_GAIN = 2 };

template <typename E, int VAR, int DK, int C, int DVH, int WSRC>
__global__ __launch_bounds__(512) void backward_chunk_kernel(BackwardParams P) {
    using LY = BwdLayout<E, DK, C, DVH>;
    constexpr int NT = 512, NW = 8;
    constexpr int PK = LY::PK, PC = LY::PC, PH = LY::PH, PF = LY::PF;
    constexpr int NB = C / 16, NTI = DK / 16, NTH = DVH / 16;
    constexpr int NSH = (NB * NTH + NW - 1) / NW;     // half-phase tiles per wave
    constexpr int NS3 = (NB * NTI + NW - 1) / NW;     // dQ~ / dK~ / dW~ tiles per wave
    constexpr int NL = NB * (NB + 1) / 2;             // dA tiles on or below the diagonal
    constexpr int NSA = (NL + NW - 1) / NW;
    constexpr bool DECAY = VAR != DELTANET;

    __shared__ __attribute__((aligned(16))) char smem[LY::TOTAL];
    E *WR = reinterpret_cast<E *>(smem + LY::OFF_WR);
    E *KR = reinterpret_cast<E *>(smem + LY::OFF_KR);
    E *TR = reinterpret_cast<E *>(smem + LY::OFF_TR);
    E *TT = reinterpret_cast<E *>(smem + LY::OFF_TT);
    E *AQT = reinterpret_cast<E *>(smem + LY::OFF_AQT);
    E *SB1 = reinterpret_cast<E *>(smem + LY::OFF_SB1);
    E *SB2 = reinterpret_cast<E *>(smem + LY::OFF_SB2);
    E *UE = reinterpret_cast<E *>(smem + LY::OFF_UE);
    E *EH = reinterpret_cast<E *>(smem + LY::OFF_EH);
    E *DOT = reinterpret_cast<E *>(smem + LY::OFF_DOT);
    E *DOH = reinterpret_cast<E *>(smem + LY::OFF_DOH);
    E *DUH = reinterpret_cast<E *>(smem + LY::OFF_DUH);
    E *DAQ = reinterpret_cast<E *>(smem + LY::OFF_DAQ);
    E *DAQT = reinterpret_cast<E *>(smem + LY::OFF_DAQT);
    E *DAK = reinterpret_cast<E *>(smem + LY::OFF_DAK);
    E *DAKT = reinterpret_cast<E *>(smem + LY::OFF_DAKT);
    E *WPT = reinterpret_cast<E *>(smem + LY::OFF_WPT);
    E *QTT = reinterpret_cast<E *>(smem + LY::OFF_QTT);
    E *KTT = reinterpret_cast<E *>(smem + LY::OFF_KTT);
    float *GAM = reinterpret_cast<float *>(smem + LY::OFF_GAM);
    float *DG = reinterpret_cast<float *>(smem + LY::OFF_DG);
    float *sm = reinterpret_cast<float *>(smem + LY::OFF_SM);
    float *s_gc = sm + LY::SM_GC, *s_dgc = sm + LY::SM_DGC, *s_sds = sm + LY::SM_SDS,
          *s_db = sm + LY::SM_DB, *s_dla = sm + LY::SM_DLA;
    int *s_flag = reinterpret_cast<int *>(sm + LY::SM_FLAG);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // records in the chain kernel's permuted column order (bf16 calls)
    const bool perm = sizeof(E) == 2 && P.rec_perm != 0;
    const int T = P.T, H = P.H, DV = P.dv;
    const int NC = (T + C - 1) / C;
    const int bh = blockIdx.x / NC, c = blockIdx.x % NC;
    const int b = bh / H, h = bh % H;
    const int c0 = c * C, L = min(C, T - c0);
    const long tok0 = ((long)b * T + c0) * H + h;      // row of (b, c0, h)
    const WsLayout LW = WsLayout::make(sizeof(E) == 2, C, DK);
    const char *rec = static_cast<const char *>(P.ws) + ((long)bh * NC + c) * LW.rec;
    const E *Sg = static_cast<const E *>(P.states) + ((long)bh * NC + c) * DK * DV;
    const E *dSg = static_cast<const E *>(P.dstates) + ((long)bh * NC + c) * DK * DV;
    const E *gq = static_cast<const E *>(P.q);
    const E *gk = static_cast<const E *>(P.k);
    const E *gv = static_cast<const E *>(P.v);
    const E *ga = static_cast<const E *>(P.alpha);
    const E *gb = static_cast<const E *>(P.beta);
    const E *gdo = static_cast<const E *>(P.dO);
    auto row = [&](int t) { return tok0 + (long)t * H; };
    // write strength of token t (isotropic KDN: derived, saved by the forward)
    auto beta_at = [&](int t) {
        return WSRC == WS_BETA_F32 ? P.beta_f32[row(t)] : to_f32(gb[row(t)]);
    };
    // diagonal KDN: the write vector is the gain w (saved by the forward),
    // and dw goes out for the variance chain instead of into dk and dbeta
    constexpr bool gw = WSRC == WS_GAIN;

    if (tid < DK) {
        s_gc[tid] = DECAY ? reinterpret_cast<const float *>(rec + LW.off_gc)[tid] : 1.f;
        s_dgc[tid] = 0.f;
        s_sds[tid] = 0.f;
    }
    if (tid < C) {
        s_db[tid] = 0.f;
        s_dla[tid] = 0.f;
    }
    if (tid == 0)
        *s_flag = 0;

    f32x4 dq3[NS3], dk3[NS3], dw3[NS3], daq[NSA], dak[NSA];
#pragma unroll
    for (int k = 0; k < NS3; ++k)
        dq3[k] = dk3[k] = dw3[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NSA; ++k)
        daq[k] = dak[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto tri = [](int x, int &bi, int &bj) {          // x-th block on or below the diagonal
        int mi = 0;
        while (x > mi) { x -= mi + 1; ++mi; }
        bi = mi;
        bj = x;
    };

    // fp32 [DK][DV] state blocks are read 4 columns at a time; NS4 units per thread
    constexpr int G4 = DVH / 4, NS4 = DK * G4 / NT;
    static_assert(NS4 * NT == DK * G4, "state staging");
    constexpr int NO4 = (C * G4 + NT - 1) / NT;
    // A half's global inputs, all issued before any is used: S and dS' of
    // its columns, dO, and V in the U-tile layout.  Rows past the sequence
    // end read the last row (every load unconditional, so they are all in
    // flight together) and are zeroed where used.
    Raw4<E> sv[NS4], dsv[NS4], dov[NO4];
    E vv[NSH][4];
    // Issued in the order of first use (S and dO, then V, then dS'), since a
    // wave's loads complete in order.
    auto load_half = [&](int jh) {
#pragma unroll
        for (int n = 0; n < NS4; ++n) {
            const int x = tid + NT * n, i = x / G4, j4 = (x % G4) * 4;
            sv[n].load(Sg + (long)i * DV + jh + j4);
        }
#pragma unroll
        for (int n = 0; n < NO4; ++n) {
            const int x = tid + NT * n, t = min(x / G4, L - 1), j4 = (x % G4) * 4;
            dov[n].load(gdo + row(t) * DV + jh + j4);
        }
#pragma unroll
        for (int k = 0; k < NSH; ++k) {
            const int tau = wv + NW * k;
            const int mt = tau / NTH, nj = tau % NTH;
            const int j = nj * 16 + (lane & 15), t0 = mt * 16 + (lane >> 4) * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vv[k][r] = gv[row(min(t0 + r, L - 1)) * DV + jh + j];
        }
#pragma unroll
        for (int n = 0; n < NS4; ++n) {
            const int x = tid + NT * n, i = x / G4, j4 = (x % G4) * 4;
            dsv[n].load(dSg + (long)i * DV + jh + j4);
        }
    };
    // S^T (or dS'^T) of the half into SB1 as [j][i]
    auto stage_t = [&](const Raw4<E> (&v)[NS4]) {
#pragma unroll
        for (int n = 0; n < NS4; ++n) {
            const int x = tid + NT * n, i = x / G4, j4 = (x % G4) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                SB1[(j4 + e) * PK + i] = from_f32<E>(v[n][e]);
        }
    };

    // ---- chunk operands from the forward record, with the first half's
    //      inputs in flight behind them
    {
        RecUnits<E, DK, C, NT> wt;
        RecUnits<E, C, DK, NT> kd;
        RecUnits<E, C, C, NT> tm, aq;
        wt.load(rec + LW.off_wdt, tid);
        kd.load(rec + LW.off_kd, tid);
        tm.load(rec + LW.off_tm, tid);
        aq.load(rec + LW.off_aqk, tid);
        load_half(0);
        // permuted (bf16 chain kernel) records hold -W~^T and -A_qk
        wt.template store<true>(WR, PK, perm ? -1.f : 1.f, tid, perm);     // W~     [s][i]
        kd.template store<false>(KR, PK, 1.f, tid, perm);    // K~     [t][i]
        tm.template store<false>(TR, PC, 1.f, tid, perm);    // T      [t][s]
        tm.template store<true>(TT, PC, 1.f, tid, perm);     // T^T    [t][s]
        aq.template store<true>(AQT, PC, perm ? -1.f : 1.f, tid, perm);    // A_qk^T [s][t]
    }
    for (int jh = 0; jh < DV; jh += DVH) {
        // ---- S^T of the half, dO^T and dO
        stage_t(sv);
#pragma unroll
        for (int n = 0; n < NO4; ++n) {
            const int x = tid + NT * n, t = x / G4, j4 = (x % G4) * 4;
            if (!((C * G4) % NT == 0 || x < C * G4)) continue;
            float d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d[e] = t < L ? dov[n][e] : 0.f;
                DOT[(j4 + e) * PC + t] = from_f32<E>(d[e]);
            }
            lds_stn<4>(DOH + t * PH + j4, d);
        }
        __syncthreads();
        // ---- U = V - K~ S  -> U^T
#pragma unroll
        for (int k = 0; k < NSH; ++k) {
            const int tau = wv + NW * k;
            if (NSH * NW != NB * NTH && tau >= NB * NTH) continue;
            const int mt = tau / NTH, nj = tau % NTH;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile_k<E, DK>(acc, KR + mt * 16 * PK, PK, SB1 + nj * 16 * PK, PK, lane);
            const int j = nj * 16 + (lane & 15), t0 = mt * 16 + (lane >> 4) * 4;
            float u[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                u[r] = (t0 + r < L ? to_f32(vv[k][r]) : 0.f) - acc[r];
            lds_stn<4>(UE + j * PC + t0, u);
        }
        __syncthreads();
        // ---- E = T U  -> E (row-major);  dS'^T of the half
#pragma unroll
        for (int k = 0; k < NSH; ++k) {
            const int tau = wv + NW * k;
            if (NSH * NW != NB * NTH && tau >= NB * NTH) continue;
            const int mt = tau / NTH, nj = tau % NTH;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile_k<E, C>(acc, TR + mt * 16 * PC, PC, UE + nj * 16 * PC, PC, lane);
            const int j = nj * 16 + (lane & 15), t0 = mt * 16 + (lane >> 4) * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                EH[(t0 + r) * PH + j] = from_f32<E>(acc[r]);
        }
        stage_t(dsv);
        __syncthreads();
        // ---- dE = A_qk^T dO + W~ dS'  -> dE^T
#pragma unroll
        for (int k = 0; k < NSH; ++k) {
            const int tau = wv + NW * k;
            if (NSH * NW != NB * NTH && tau >= NB * NTH) continue;
            const int ms = tau / NTH, nj = tau % NTH;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile_k<E, C>(acc, AQT + ms * 16 * PC, PC, DOT + nj * 16 * PC, PC, lane);
            mma_tile_k<E, DK>(acc, WR + ms * 16 * PK, PK, SB1 + nj * 16 * PK, PK, lane);
            float e4[4] = {acc[0], acc[1], acc[2], acc[3]};
            lds_stn<4>(UE + (nj * 16 + (lane & 15)) * PC + ms * 16 + (lane >> 4) * 4, e4);
        }
        __syncthreads();
        // ---- dU = T^T dE  -> dv and dU (row-major);  S and dS' of the half
        //      (row-major) and sum_j S dS'
#pragma unroll
        for (int k = 0; k < NSH; ++k) {
            const int tau = wv + NW * k;
            if (NSH * NW != NB * NTH && tau >= NB * NTH) continue;
            const int mt = tau / NTH, nj = tau % NTH;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile_k<E, C>(acc, TT + mt * 16 * PC, PC, UE + nj * 16 * PC, PC, lane);
            const int j = nj * 16 + (lane & 15), t0 = mt * 16 + (lane >> 4) * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                DUH[(t0 + r) * PH + j] = from_f32<E>(acc[r]);
                if (t0 + r < L)
                    P.dv_[row(t0 + r) * DV + jh + j] = acc[r];
            }
        }
        {
#pragma unroll
            for (int n = 0; n < NS4; ++n) {
                const int x = tid + NT * n, i = x / G4, j4 = (x % G4) * 4;
                sv[n].store(SB1 + i * PH + j4);
                dsv[n].store(SB2 + i * PH + j4);
                if (DECAY) {
                    // sum over the G4 lanes of key channel i, then one atomic
                    float p = sv[n][0] * dsv[n][0] + sv[n][1] * dsv[n][1] +
                              sv[n][2] * dsv[n][2] + sv[n][3] * dsv[n][3];
                    if constexpr (G4 == 16) {
                        p = row16_sum_last(p);
                        if (lane % 16 == 15)
                            atomicAdd(&s_sds[i], p);
                    } else {
#pragma unroll
                        for (int off = G4 / 2; off >= 1; off >>= 1)
                            p += __shfl_xor(p, off, WAVE);
                        if (lane % G4 == 0)
                            atomicAdd(&s_sds[i], p);
                    }
                }
            }
        }
        if (jh + DVH < DV)
            load_half(jh + DVH);                       // in flight during the sums
        __syncthreads();
        // ---- sums over the half's columns
#pragma unroll
        for (int k = 0; k < NS3; ++k) {
            const int tau = wv + NW * k;
            if (NS3 * NW != NB * NTI && tau >= NB * NTI) continue;
            const int mt = tau / NTI, ni = tau % NTI;
            mma_tile_k<E, DVH>(dq3[k], DOH + mt * 16 * PH, PH, SB1 + ni * 16 * PH, PH, lane);
            mma_tile_k<E, DVH>(dk3[k], DUH + mt * 16 * PH, PH, SB1 + ni * 16 * PH, PH, lane);
            mma_tile_k<E, DVH>(dw3[k], EH + mt * 16 * PH, PH, SB2 + ni * 16 * PH, PH, lane);
        }
#pragma unroll
        for (int k = 0; k < NSA; ++k) {
            const int x = wv + NW * k;
            if (x >= NL) continue;
            int bi, bj;
            tri(x, bi, bj);
            mma_tile_k<E, DVH>(daq[k], DOH + bi * 16 * PH, PH, EH + bj * 16 * PH, PH, lane);
            mma_tile_k<E, DVH>(dak[k], DUH + bi * 16 * PH, PH, EH + bj * 16 * PH, PH, lane);
        }
        __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < NS3; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dk3[k][r] = -dk3[k][r];

    // ---- decays gamma_t per channel; W'^T = (w / gamma)^T, Q~^T, K~^T;
    //      the dA matrices (masked) and their transposes; sum_s W~ dW~
    // decays into GAM (a_t per channel; 1 past the sequence end)
    constexpr int GK4 = DK / 4, NK4 = C * GK4 / NT;
    static_assert(NK4 * NT == C * GK4, "chunk tile units");
    static_assert(NS3 * NW == NB * NTI, "one element set per thread");
    // The thread's elements of the [C][DK] tiles (tile tau = wv + NW k, row r:
    // t = mt 16 + (lane >> 4) 4 + r, i = ni 16 + (lane & 15)): k, q and the
    // gain (diagonal KDN) or beta, read once with the decays for the scaled
    // operands and the elementwise step.
    float ek[NS3][4], eq[NS3][4], ew[NS3][4];
    {
        float a4[NK4][4];
#pragma unroll
        for (int n = 0; n < NK4; ++n) {
            const int x = tid + NT * n, t = min(x / GK4, L - 1), i4 = (x % GK4) * 4;
            a4[n][0] = a4[n][1] = a4[n][2] = a4[n][3] = 1.f;
            if (VAR == KDA)
                gload4(ga + row(t) * DK + i4, a4[n]);
            if (VAR == GATED_DELTANET)
                a4[n][0] = a4[n][1] = a4[n][2] = a4[n][3] = to_f32(ga[row(t)]);
        }
#pragma unroll
        for (int k = 0; k < NS3; ++k) {
            const int tau = wv + NW * k;
            const int mt = tau / NTI, ni = tau % NTI;
            const int i = ni * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = min(mt * 16 + (lane >> 4) * 4 + r, L - 1);
                ek[k][r] = to_f32(gk[row(t) * DK + i]);
                eq[k][r] = to_f32(gq[row(t) * DK + i]);
                ew[k][r] = gw ? P.w_f32[row(t) * DK + i] : beta_at(t);
            }
        }
#pragma unroll
        for (int n = 0; n < NK4; ++n) {
            const int x = tid + NT * n, t = x / GK4, i4 = (x % GK4) * 4;
            const bool in = t < L;
            *reinterpret_cast<float4 *>(GAM + t * PF + i4) =
                make_float4(in ? a4[n][0] : 1.f, in ? a4[n][1] : 1.f, in ? a4[n][2] : 1.f,
                            in ? a4[n][3] : 1.f);
        }
    }
    for (int x = tid; x < C * C; x += NT) {            // blocks above the diagonal
        const int t = x / C, s = x % C;
        if ((s >> 4) > (t >> 4)) {
            DAQ[t * PC + s] = DAK[t * PC + s] = from_f32<E>(0.f);
            DAQT[s * PC + t] = DAKT[s * PC + t] = from_f32<E>(0.f);
        }
    }
#pragma unroll
    for (int k = 0; k < NSA; ++k) {
        const int x = wv + NW * k;
        if (x >= NL) continue;
        int bi, bj;
        tri(x, bi, bj);
        const int s = bj * 16 + (lane & 15), t0 = bi * 16 + (lane >> 4) * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + r;
            const E vq = from_f32<E>(s <= t ? daq[k][r] : 0.f);
            const E vk = from_f32<E>(s < t ? -dak[k][r] : 0.f);
            DAQ[t * PC + s] = vq;
            DAQT[s * PC + t] = vq;
            DAK[t * PC + s] = vk;
            DAKT[s * PC + t] = vk;
        }
    }
    if (DECAY) {
        // sum_s W~_s,i dW~_s,i (the W~ term of d log gamma_C)
#pragma unroll
        for (int k = 0; k < NS3; ++k) {
            const int tau = wv + NW * k;
            if (NS3 * NW != NB * NTI && tau >= NB * NTI) continue;
            const int mt = tau / NTI, ni = tau % NTI;
            const int i = ni * 16 + (lane & 15), t0 = mt * 16 + (lane >> 4) * 4;
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc += to_f32(WR[(t0 + r) * PK + i]) * dw3[k][r];
            acc += __shfl_xor(acc, 16, WAVE);
            acc += __shfl_xor(acc, 32, WAVE);
            if (lane < 16)
                atomicAdd(&s_dgc[i], acc);
        }
    }
    __syncthreads();
    // gamma_t = prod_{r <= t} a_r per channel, in place
    if (DECAY && tid < DK) {
        const int i = tid;
        float a[C];
#pragma unroll
        for (int t = 0; t < C; ++t)
            a[t] = GAM[t * PF + i];
        float g = 1.f;
#pragma unroll
        for (int t = 0; t < C; ++t) {
            g *= a[t];
            GAM[t * PF + i] = g;
        }
        if (!(g >= KDN_DECAY_FLOOR))
            *s_flag = 1;
    }
    __syncthreads();
    // W'^T = (w / gamma)^T, Q~^T = (gamma q)^T, K~^T = (gamma k)^T, four
    // consecutive tokens of one channel per store
#pragma unroll
    for (int k = 0; k < NS3; ++k) {
        const int tau = wv + NW * k;
        const int mt = tau / NTI, ni = tau % NTI;
        const int i = ni * 16 + (lane & 15), t0 = mt * 16 + (lane >> 4) * 4;
        float wp[4], qt[4], kt[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (t0 + r >= L)                           // rows past the end: zero
                ek[k][r] = eq[k][r] = ew[k][r] = 0.f;
            const float g = GAM[(t0 + r) * PF + i];
            const float w = gw ? ew[k][r] : ew[k][r] * ek[k][r];
            wp[r] = g > 0.f ? w / g : 0.f;
            qt[r] = g * eq[k][r];
            kt[r] = g * ek[k][r];
        }
        lds_stn<4>(WPT + i * PC + t0, wp);
        lds_stn<4>(QTT + i * PC + t0, qt);
        lds_stn<4>(KTT + i * PC + t0, kt);
    }
    __syncthreads();
    const bool exact = *s_flag != 0;

    // ---- decay-scaled products (or their exact elementwise sums)
    if (!exact) {
#pragma unroll
        for (int k = 0; k < NS3; ++k) {
            const int tau = wv + NW * k;
            if (NS3 * NW != NB * NTI && tau >= NB * NTI) continue;
            const int mt = tau / NTI, ni = tau % NTI;
            const int i0 = ni * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dw3[k][r] *= s_gc[i0];
            mma_tile_k<E, C>(dq3[k], DAQ + mt * 16 * PC, PC, WPT + ni * 16 * PC, PC, lane);
            mma_tile_k<E, C>(dk3[k], DAK + mt * 16 * PC, PC, WPT + ni * 16 * PC, PC, lane);
            mma_tile_k<E, C>(dw3[k], DAKT + mt * 16 * PC, PC, KTT + ni * 16 * PC, PC, lane);
            mma_tile_k<E, C>(dw3[k], DAQT + mt * 16 * PC, PC, QTT + ni * 16 * PC, PC, lane);
        }
    } else {
        // Exact: with R(t, s) = prod_{s < r <= t} a_r (per channel),
        //   dq_t = gamma_t dQ~S_t + sum_{s<=t} dA_qk[t,s] w_s R(t,s),
        //   gamma_t dK~_t likewise with dA_kk (s < t),
        //   dw_s = R(C-1,s) dW~_s + sum_{t>s} dA_kk[t,s] k_t R(t,s)
        //          + sum_{t>=s} dA_qk[t,s] q_t R(t,s),
        // stored already scaled (dq3 <- dq, dk3 <- gamma dK~, dw3 <- dw).
        auto dec = [&](int t, int i) {
            if (t >= L) return 1.f;
            return VAR == GATED_DELTANET ? to_f32(ga[row(t)])
                 : (VAR == KDA ? to_f32(ga[row(t) * DK + i]) : 1.f);
        };
        auto wval = [&](int s, int i) {
            if (s >= L) return 0.f;
            return gw ? P.w_f32[row(s) * DK + i] : beta_at(s) * to_f32(gk[row(s) * DK + i]);
        };
#pragma unroll
        for (int k = 0; k < NS3; ++k) {
            const int tau = wv + NW * k;
            if (NS3 * NW != NB * NTI && tau >= NB * NTI) continue;
            const int mt = tau / NTI, ni = tau % NTI;
            const int i = ni * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = mt * 16 + (lane >> 4) * 4 + r;
                const float g = GAM[t * PF + i];
                float xq = g * dq3[k][r], xk = g * dk3[k][r];
                float R = 1.f;
                for (int s = t; s >= 0; --s) {
                    const float w = wval(s, i);
                    xq += to_f32(DAQ[t * PC + s]) * w * R;
                    if (s < t)
                        xk += to_f32(DAK[t * PC + s]) * w * R;
                    R *= dec(s, i);
                }
                float rc = 1.f;                           // R(C-1, t)
                for (int u = t + 1; u < C; ++u)
                    rc *= dec(u, i);
                float xw = rc * dw3[k][r];
                R = 1.f;
                for (int u = t; u < C; ++u) {
                    if (u > t)
                        R *= dec(u, i);
                    const float kk = u < L ? to_f32(gk[row(u) * DK + i]) : 0.f;
                    const float qq = u < L ? to_f32(gq[row(u) * DK + i]) : 0.f;
                    if (u > t)
                        xw += to_f32(DAK[u * PC + t]) * kk * R;
                    xw += to_f32(DAQ[u * PC + t]) * qq * R;
                }
                dq3[k][r] = xq;
                dk3[k][r] = xk;
                dw3[k][r] = xw;
            }
        }
    }
    __syncthreads();                                   // dA, W'^T read; DG overwrites them

    // ---- elementwise: dq, dk, dbeta, d log gamma
#pragma unroll
    for (int k = 0; k < NS3; ++k) {
        const int tau = wv + NW * k;
        if (NS3 * NW != NB * NTI && tau >= NB * NTI) continue;
        const int mt = tau / NTI, ni = tau % NTI;
        const int i = ni * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = mt * 16 + (lane >> 4) * 4 + r;
            const bool in = t < L;
            const float g = GAM[t * PF + i];
            const float kk = ek[k][r], qq = eq[k][r];
            const float bt = gw ? 0.f : ew[k][r];
            const float wv = gw ? ew[k][r] : bt * kk;
            const float dq = exact ? dq3[k][r] : g * dq3[k][r];
            const float dkd = exact ? dk3[k][r] : g * dk3[k][r];
            const float dw = exact ? dw3[k][r] : (g > 0.f ? dw3[k][r] / g : 0.f);
            if (in) {
                P.dq[row(t) * DK + i] = dq;
                P.dk_[row(t) * DK + i] = dkd + bt * dw;
                if (gw)
                    P.dw_out[row(t) * DK + i] = dw;
            }
            // dbeta (diagonal KDN: sum w dw) over the 16 channels of the row:
            // a DPP row sum, then one atomic per row
            const float db = row16_sum_last((gw ? wv : kk) * dw);
            if ((lane & 15) == 15)
                atomicAdd(&s_db[t], db);
            if (DECAY)
                DG[t * PF + i] = kk * dkd + qq * dq - wv * dw;
        }
    }
    __syncthreads();
    // ---- d log alpha: reverse sum over the chunk's tokens, plus the gamma_C terms
    if (VAR == KDA && tid < DK) {
        const int i = tid;
        float dg[C];
#pragma unroll
        for (int t = 0; t < C; ++t)
            dg[t] = DG[t * PF + i];
        float acc = s_dgc[i] + s_gc[i] * s_sds[i];
#pragma unroll
        for (int t = C - 1; t >= 0; --t) {
            acc += dg[t];
            if (t < L)
                P.dla[row(t) * DK + i] = acc;
        }
    }
    if (VAR == GATED_DELTANET) {
        // one decay per token: 8 lanes per token sum its channels (a row of 8
        // lanes reads 32 consecutive floats), a DPP sum over the 8; then a
        // suffix sum over the tokens across the lanes of wave 0
        static_assert(DK % 32 == 0 && C * 8 <= NT, "row sums");
        if (tid < C * 8) {
            const int t = tid >> 3, part = tid & 7;
            float x = 0.f;
#pragma unroll
            for (int q = 0; q < DK / 32; ++q) {
                const float4 v = *reinterpret_cast<const float4 *>(DG + t * PF + part * 4 + 32 * q);
                x += (v.x + v.y) + (v.z + v.w);
            }
            x = row8_sum_last(x);
            if (part == 7)
                s_dla[t] = x;
        }
        __syncthreads();
        if (wv == 0) {
            float gcs = 0.f;
            for (int i = lane; i < DK; i += WAVE)
                gcs += s_dgc[i] + s_gc[i] * s_sds[i];
            gcs = wave_sum(gcs);
            float v = lane < C ? s_dla[lane] : 0.f;
#pragma unroll
            for (int off = 1; off < WAVE; off <<= 1) {
                const float y = __shfl_down(v, off, WAVE);
                if (lane + off < WAVE)
                    v += y;
            }
            if (lane < L)
                P.dla[row(lane)] = v + gcs;
        }
    }
    float *const dbo = gw ? P.wdw : P.dbeta;
    if (tid < L && dbo)
        dbo[row(tid)] = s_db[tid];
}

// ---------------------------------------------------------------------------
// Isotropic KDN: the adjoint of the head-variance chain.  Per token, forward
//   p- = a2 p + xm,  s = r + p- kk,  beta = p- / s,  den = r + m p- kk,
//   p' = p- r / den   (m = mu / d_k; s = 0: beta = 0; den = 0: p' = p-),
// the gradient of the variance before the token is affine in the gradient dp
// of p' once dbeta is known (the memory part of the backward gives it):
//   dp- = dbeta r / s^2 + dp c,  c = r^2 / den^2 (1 if den = 0),
//   d(previous p) = a2 dp- = A dp + Bc,  A = a2 c,  Bc = a2 dbeta r / s^2.
// Kernel 1 composes each chunk's token maps; kernel 2 runs the chunk maps
// backwards from dp_out, giving dp at every chunk end and dp0; kernel 3
// forms every token's dp and its gradients:
//   dkk = -dbeta p-^2 / s^2 - dp m p-^2 r / den^2,
//   dr = -dbeta p- / s^2 + dp m p-^2 kk / den^2,  da2 = dp- p,  dxm = dp-,
// added to dk (2 dkk k), d log alpha (2 da2 a^2 / d_k) and written to dxi
// (dxm / d_k) and dr.
// ---------------------------------------------------------------------------
struct ChainTok {
    float a2, xm, kk, r, pp, pm, s, den, db, A, Bc;
};

// Lane t of a wave: token t of chunk c of head bh (identity past the end).
// The variance before each token comes from the chunk-start variance by the
// same scan of the token maps as the forward pass.
__device__ __forceinline__ ChainTok chain_token(const BackwardParams &P, int bh, int c,
                                                int NC, int C, int lane) {
    const int T = P.T, H = P.H;
    const int b = bh / H, h = bh % H, c0 = c * C, L = min(C, T - c0);
    const bool in = lane < L;
    ChainTok x;
    const float4 st = in ? reinterpret_cast<const float4 *>(P.ws_stat)[((long)bh * NC + c) * C + lane]
                         : make_float4(1.f, 0.f, 0.f, 1.f);
    x.a2 = st.x; x.xm = st.y; x.kk = st.z; x.r = st.w;
    const float mdk = P.mu * (1.f / P.dk);
    Map2 M = variance_step_map(x.a2, x.xm, mdk * x.kk, x.r);
    M.rescale();
    for (int off = 1; off < C; off <<= 1) {
        const float ya = __shfl_up(M.a, off, WAVE), yb = __shfl_up(M.b, off, WAVE);
        const float yc = __shfl_up(M.c, off, WAVE), yd = __shfl_up(M.d, off, WAVE);
        if (lane >= off) {
            M.before(ya, yb, yc, yd);
            M.rescale();
        }
    }
    const float p0 = P.ws_p0[(long)bh * NC + c];
    const float pt = M.apply(p0);
    float pp = __shfl_up(pt, 1, WAVE);
    if (lane == 0)
        pp = p0;
    x.pp = pp;
    x.pm = fmaf(x.a2, pp, x.xm);
    x.s = fmaf(x.pm, x.kk, x.r);
    x.den = fmaf(mdk * x.pm, x.kk, x.r);
    x.db = in ? P.dbeta[((long)b * T + c0 + lane) * H + h] : 0.f;
    const float cc = x.den != 0.f ? (x.r * x.r) / (x.den * x.den) : 1.f;
    x.A = x.a2 * cc;
    x.Bc = x.s != 0.f ? x.a2 * x.db * x.r / (x.s * x.s) : 0.f;
    if (!in) {
        x.A = 1.f;
        x.Bc = 0.f;
    }
    return x;
}

// Suffix composition over the lanes: lane t gets f_t o f_{t+1} o ... o f_{C-1}
// (f applied last-token first).
__device__ __forceinline__ void chain_suffix(float &A, float &Bc, int C, int lane) {
    for (int off = 1; off < C; off <<= 1) {
        const float ya = __shfl_down(A, off, WAVE), yb = __shfl_down(Bc, off, WAVE);
        if (lane + off < C) {
            Bc = fmaf(A, yb, Bc);
            A *= ya;
        }
    }
}

// Kernel 1: one wave per (head, chunk), chunk maps to chain_map [bh][c][2].
__global__ __launch_bounds__(256) void iso_chain_map_kernel(BackwardParams P) {
    const int C = P.chunk, NC = (P.T + C - 1) / C;
    const long unit = (long)blockIdx.x * 4 + threadIdx.x / WAVE;
    if (unit >= (long)P.B * P.H * NC)
        return;
    const int lane = threadIdx.x & (WAVE - 1);
    const int bh = (int)(unit / NC), c = (int)(unit % NC);
    ChainTok x = chain_token(P, bh, c, NC, C, lane);
    float A = x.A, Bc = x.Bc;
    chain_suffix(A, Bc, C, lane);
    if (lane == 0) {
        P.chain_map[unit * 2] = A;
        P.chain_map[unit * 2 + 1] = Bc;
    }
}

// Kernel 3: one wave per (head, chunk): every token's dp, its scalar
// gradients, then the per-channel ones (lanes over the channels).
template <typename E>
__global__ __launch_bounds__(256) void iso_chain_grad_kernel(BackwardParams P) {
    __shared__ float sg[4][3][64];                 // per wave: dkk, da2, dxm of each token
    const int C = P.chunk, NC = (P.T + C - 1) / C;
    const int w = threadIdx.x / WAVE;
    const long unit = (long)blockIdx.x * 4 + w;
    if (unit >= (long)P.B * P.H * NC)
        return;
    const int lane = threadIdx.x & (WAVE - 1);
    const int bh = (int)(unit / NC), c = (int)(unit % NC);
    const int T = P.T, H = P.H, DK = P.dk;
    const int b = bh / H, h = bh % H, c0 = c * C, L = min(C, T - c0);
    ChainTok x = chain_token(P, bh, c, NC, C, lane);
    float A = x.A, Bc = x.Bc;
    chain_suffix(A, Bc, C, lane);
    // dp of token t = (f_{t+1} o ... o f_{C-1})(dp at the chunk end)
    float An = __shfl_down(A, 1, WAVE), Bn = __shfl_down(Bc, 1, WAVE);
    if (lane + 1 >= C) {
        An = 1.f;
        Bn = 0.f;
    }
    const float dpe = P.chain_dp[(long)bh * NC + c];
    const float dp = fmaf(An, dpe, Bn);
    const float mdk = P.mu * (1.f / DK);
    const float s2 = x.s * x.s, d2 = x.den * x.den, pm2 = x.pm * x.pm;
    float dpm = 0.f, dkk = 0.f, dr = 0.f;
    if (x.s != 0.f) {
        dpm += x.db * x.r / s2;
        dkk -= x.db * pm2 / s2;
        dr -= x.db * x.pm / s2;
    }
    if (x.den != 0.f) {
        dpm += dp * x.r * x.r / d2;
        dkk -= dp * mdk * pm2 * x.r / d2;
        dr += dp * mdk * pm2 * x.kk / d2;
    } else {
        dpm += dp;
    }
    const long tok = ((long)b * T + c0 + lane) * H + h;
    if (lane < L)
        P.dr[tok] = dr;
    if (lane < C) {
        sg[w][0][lane] = dkk;
        sg[w][1][lane] = dpm * x.pp;                 // da2
        sg[w][2][lane] = dpm;                        // dxm
    }
    __builtin_amdgcn_wave_barrier();
    const E *gk = static_cast<const E *>(P.k);
    const E *ga = static_cast<const E *>(P.alpha);
    const float inv = 1.f / DK;
    for (int t = 0; t < L; ++t) {
        const long rt = ((long)b * T + c0 + t) * H + h;
        const float tkk = sg[w][0][t], ta2 = sg[w][1][t], txm = sg[w][2][t];
        for (int i = lane; i < DK; i += WAVE) {
            const float kv = to_f32(gk[rt * DK + i]), av = to_f32(ga[rt * DK + i]);
            P.dxi[rt * DK + i] = txm * inv;
            P.dk_[rt * DK + i] += 2.f * tkk * kv;
            P.dla[rt * DK + i] += 2.f * ta2 * av * av * inv;
        }
    }
}

// ---------------------------------------------------------------------------
// Diagonal KDN: the adjoint of the per-channel variance chain.  Per token,
// forward (channel i; s couples the channels):
//   p-_i = a_i^2 p_i + xi_i,  s = r + sum_i p-_i k_i^2,  w_i = p-_i k_i / s,
//   den_i = r + mu p-_i k_i^2,  p'_i = p-_i r / den_i
// (s = 0: w = 0; den_i = 0: p'_i = p-_i).  With dw from the memory part,
//   du_i = dw_i / s,  ds = -sum_i dw_i w_i / s          (0 if s = 0)
//   dp-_i = du_i k_i + ds k_i^2 + dp_i c_i,  c_i = r^2 / den_i^2 (1 if 0)
//   d(previous p_i) = a_i^2 dp-_i,
// affine in dp_i: A = a^2 c, Bc = a^2 (du k + ds k^2).  The gradients:
//   dk_i += du_i p-_i + 2 ds p-_i k_i - 2 dp_i mu p-_i^2 r k_i / den_i^2,
//   dr = ds + sum_i dp_i mu p-_i^2 k_i^2 / den_i^2,
//   d log alpha_i += 2 a_i^2 p_i dp-_i,  dxi_i = dp-_i.
// The forward pass saved 1/s per token and the memory part sum_i w_i dw_i,
// so given those the channels are independent: one wave per (head, chunk),
// lane l holding channels NJ l .. NJ l + NJ - 1, every token's inputs read a
// group of tokens ahead so the loads stay off the sequential chain.
// ---------------------------------------------------------------------------
template <int NJ, typename E>
__device__ __forceinline__ void ld_ch(const E *p, float (&x)[NJ]) {
    if constexpr (NJ == 1) {
        x[0] = to_f32(p[0]);
    } else if constexpr (sizeof(E) == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t *>(p);
        x[0] = __uint_as_float(u << 16);
        x[1] = __uint_as_float(u & 0xffff0000u);
    } else {
        const float2 f = *reinterpret_cast<const float2 *>(p);
        x[0] = f.x;
        x[1] = f.y;
    }
}
template <int NJ>
__device__ __forceinline__ void st_ch(float *p, const float (&x)[NJ]) {
    if constexpr (NJ == 1)
        p[0] = x[0];
    else
        *reinterpret_cast<float2 *>(p) = make_float2(x[0], x[1]);
}
__device__ __forceinline__ float lane_bcast(float x, int t) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), t));
}

// Unit (head, chunk) of a diagonal-chain wave, with lane t holding token t's
// observation noise, 1/s and ds (1, 0, 0 past the chunk's end).
struct DiagUnit {
    long unit, tok0;
    int L;
    float r, invs, ds;
};
template <typename E>
__device__ __forceinline__ bool diag_unit(const BackwardParams &P, int C, DiagUnit &U) {
    const int NC = (P.T + C - 1) / C;
    U.unit = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (U.unit >= (long)P.B * P.H * NC)
        return false;
    const int lane = threadIdx.x & (WAVE - 1);
    const int bh = (int)(U.unit / NC), c = (int)(U.unit % NC);
    const int b = bh / P.H, h = bh % P.H, c0 = c * C;
    U.L = min(C, P.T - c0);
    U.tok0 = ((long)b * P.T + c0) * P.H + h;
    U.r = 1.f;
    U.invs = 0.f;
    U.ds = 0.f;
    if (lane < U.L) {
        const long row = U.tok0 + (long)lane * P.H;
        U.r = to_f32(static_cast<const E *>(P.r)[row]);
        U.invs = P.invs[row];
        U.ds = -U.invs * P.wdw[row];
    }
    return true;
}

// Kernel 2 (both KDN variants): the chain's chunk maps composed from the
// last chunk back.  Sequence s (a head, or a head's key channel: nch per
// head) has NC maps, map c at chain_map[((s / nch) NC + c) nch + s % nch]
// (pairs A, B: dp before chunk c = A dp after it + B).  One wave per
// sequence takes 64 chunks at a time: a suffix composition over the lanes
// gives every chunk-end gradient of the block from the one at its end.
__global__ __launch_bounds__(256) void chain_scan_kernel(BackwardParams P, int nch) {
    const long s = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (s >= (long)P.B * P.H * nch)
        return;
    const int lane = threadIdx.x & (WAVE - 1);
    const long bh = s / nch;
    const int i = (int)(s % nch);
    const int NC = (P.T + P.chunk - 1) / P.chunk;
    const float2 *maps = reinterpret_cast<const float2 *>(P.chain_map);
    float carry = P.dp_out ? P.dp_out[s] : 0.f;
    for (int hi = NC; hi > 0; hi -= WAVE) {
        const int c = hi - WAVE + lane;
        const long u = (bh * NC + c) * nch + i;
        float A = 1.f, Bc = 0.f;
        if (c >= 0) {
            const float2 m = maps[u];
            A = m.x;
            Bc = m.y;
        }
        chain_suffix(A, Bc, WAVE, lane);           // lane l: m_l o ... o m_63
        float EA = __shfl_down(A, 1, WAVE), EB = __shfl_down(Bc, 1, WAVE);
        if (lane == WAVE - 1) {
            EA = 1.f;
            EB = 0.f;
        }
        if (c >= 0)
            P.chain_dp[u] = fmaf(EA, carry, EB);
        carry = fmaf(lane_bcast(A, 0), carry, lane_bcast(Bc, 0));
    }
    if (lane == 0 && P.dp0)
        P.dp0[s] = carry;
}

// Kernel 1: the chain through the chunk from its start variance (the same
// arithmetic as the forward pass), saving the variance before each token,
// and the chunk map F = f_0 o ... o f_{L-1} composed in token order, to
// chain_map [bh][c][dk][2].
template <typename E, int DK, int C>
__global__ __launch_bounds__(256) void diag_chain_map_kernel(BackwardParams P) {
    constexpr int NJ = DK / WAVE, G = 8;
    DiagUnit U;
    if (!diag_unit<E>(P, C, U))
        return;
    const int i0 = (threadIdx.x & (WAVE - 1)) * NJ;
    const long H = P.H;
    const E *gk = static_cast<const E *>(P.k);
    const E *ga = static_cast<const E *>(P.alpha);
    const E *gx = static_cast<const E *>(P.xi);
    const float mu = P.mu;
    float p[NJ], FA[NJ], FB[NJ];
    ld_ch<NJ>(P.ws_p0 + U.unit * DK + i0, p);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        FA[j] = 1.f;
        FB[j] = 0.f;
    }
#pragma unroll 1
    for (int tb = 0; tb < U.L; tb += G) {
        float kk[G][NJ], aa[G][NJ], xx[G][NJ], dw[G][NJ];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const long row = U.tok0 + (long)(tb + g) * H;
            if (tb + g < U.L) {
                ld_ch<NJ>(gk + row * DK + i0, kk[g]);
                ld_ch<NJ>(ga + row * DK + i0, aa[g]);
                ld_ch<NJ>(gx + row * DK + i0, xx[g]);
                ld_ch<NJ>(P.dw_out + row * DK + i0, dw[g]);
            } else {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    kk[g][j] = 0.f; aa[g][j] = 1.f; xx[g][j] = 0.f; dw[g][j] = 0.f;
                }
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t = tb + g;
            const float r = lane_bcast(U.r, t), invs = lane_bcast(U.invs, t);
            const float ds = lane_bcast(U.ds, t);
            if (t < U.L)
                st_ch<NJ>(P.pp + (U.tok0 + (long)t * H) * DK + i0, p);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float k = kk[g][j], a2 = aa[g][j] * aa[g][j];
                const float pm = fmaf(a2, p[j], xx[g][j]);
                const float den = fmaf(mu * k * k, pm, r);
                p[j] = den != 0.f ? pm * r * fast_rcp(den) : pm;
                const float cc = den != 0.f ? (r * r) / (den * den) : 1.f;
                const float du = dw[g][j] * invs;
                FB[j] = fmaf(FA[j], a2 * fmaf(ds * k, k, du * k), FB[j]);
                FA[j] *= a2 * cc;
            }
        }
    }
    float *dst = P.chain_map + (U.unit * DK + i0) * 2;
    if constexpr (NJ == 2)
        *reinterpret_cast<float4 *>(dst) = make_float4(FA[0], FB[0], FA[1], FB[1]);
    else
        *reinterpret_cast<float2 *>(dst) = make_float2(FA[0], FB[0]);
}

// Kernel 3: from dp at the chunk end, the tokens in reverse: every token's
// dp and gradients (dk and d log alpha added to the memory part's).
template <typename E, int DK, int C>
__global__ __launch_bounds__(256) void diag_chain_grad_kernel(BackwardParams P) {
    constexpr int NJ = DK / WAVE, G = 4;
    DiagUnit U;
    if (!diag_unit<E>(P, C, U))
        return;
    const int lane = threadIdx.x & (WAVE - 1), i0 = lane * NJ;
    const long H = P.H;
    const E *gk = static_cast<const E *>(P.k);
    const E *ga = static_cast<const E *>(P.alpha);
    const E *gx = static_cast<const E *>(P.xi);
    const float mu = P.mu;
    float dp[NJ];
    ld_ch<NJ>(P.chain_dp + U.unit * DK + i0, dp);
#pragma unroll 1
    for (int tb = (U.L - 1) / G * G; tb >= 0; tb -= G) {
        float kk[G][NJ], aa[G][NJ], xx[G][NJ], dw[G][NJ], pv[G][NJ], gk_[G][NJ], gl[G][NJ];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const long o = (U.tok0 + (long)(tb + g) * H) * DK + i0;
            if (tb + g < U.L) {
                ld_ch<NJ>(gk + o, kk[g]);
                ld_ch<NJ>(ga + o, aa[g]);
                ld_ch<NJ>(gx + o, xx[g]);
                ld_ch<NJ>(P.dw_out + o, dw[g]);
                ld_ch<NJ>(P.pp + o, pv[g]);
                ld_ch<NJ>(P.dk_ + o, gk_[g]);
                ld_ch<NJ>(P.dla + o, gl[g]);
            } else {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    kk[g][j] = 0.f; aa[g][j] = 1.f; xx[g][j] = 0.f; dw[g][j] = 0.f;
                    pv[g][j] = 0.f; gk_[g][j] = 0.f; gl[g][j] = 0.f;
                }
            }
        }
        float drs[G];
#pragma unroll
        for (int g = G - 1; g >= 0; --g) {
            const int t = tb + g;
            const float r = lane_bcast(U.r, t), invs = lane_bcast(U.invs, t);
            const float ds = lane_bcast(U.ds, t);
            float dxi[NJ];
            drs[g] = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float k = kk[g][j], a2 = aa[g][j] * aa[g][j], pp = pv[g][j];
                const float pm = fmaf(a2, pp, xx[g][j]);
                const float den = fmaf(mu * k * k, pm, r);
                const float du = dw[g][j] * invs;
                float dpm = fmaf(ds * k, k, du * k);
                float dki = fmaf(2.f * ds * pm, k, du * pm);
                if (den != 0.f) {
                    const float q = dp[j] / (den * den);
                    dpm = fmaf(q, r * r, dpm);
                    dki -= 2.f * q * mu * pm * pm * r * k;
                    drs[g] = fmaf(q * mu * pm * pm, k * k, drs[g]);
                } else {
                    dpm += dp[j];
                }
                gk_[g][j] += dki;
                gl[g][j] = fmaf(2.f * a2 * pp, dpm, gl[g][j]);
                dxi[j] = dpm;
                dp[j] = a2 * dpm;
            }
            if (t < U.L) {
                const long o = (U.tok0 + (long)t * H) * DK + i0;
                st_ch<NJ>(P.dk_ + o, gk_[g]);
                st_ch<NJ>(P.dla + o, gl[g]);
                st_ch<NJ>(P.dxi + o, dxi);
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t = tb + g;
            const float x = wave_sum(drs[g]);
            if (lane == 0 && t < U.L)
                P.dr[U.tok0 + (long)t * H] = lane_bcast(U.ds, t) + x;
        }
    }
}

template <typename E, int DK, int C>
static hipError_t launch_diag_chain(const BackwardParams &P, hipStream_t st) {
    const long bh = (long)P.B * P.H, nc = (P.T + C - 1) / C;
    const dim3 g((unsigned)((bh * nc + 3) / 4)), blk(256);
    if (nc > 0) {
        hipLaunchKernelGGL((diag_chain_map_kernel<E, DK, C>), g, blk, 0, st, P);
        if (hipError_t e = hipGetLastError())
            return e;
    }
    hipLaunchKernelGGL(chain_scan_kernel, dim3((unsigned)((bh * DK + 3) / 4)), dim3(256), 0, st,
                       P, DK);
    if (hipError_t e = hipGetLastError())
        return e;
    if (nc > 0)
        hipLaunchKernelGGL((diag_chain_grad_kernel<E, DK, C>), g, blk, 0, st, P);
    return hipGetLastError();
}

template <typename E>
static hipError_t launch_diag_chain_e(const BackwardParams &P, hipStream_t st) {
    if (P.dk == 128 && P.chunk == 64) return launch_diag_chain<E, 128, 64>(P, st);
    if (P.dk == 128 && P.chunk == 32) return launch_diag_chain<E, 128, 32>(P, st);
    if (P.dk == 64 && P.chunk == 64) return launch_diag_chain<E, 64, 64>(P, st);
    if (P.dk == 64 && P.chunk == 32) return launch_diag_chain<E, 64, 32>(P, st);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
template <typename E, int VAR, int DK, int C>
static hipError_t launch_bwd_vc(const BackwardParams &P, hipStream_t st) {
    const long heads = (long)P.B * P.H;
    const long nc = (P.T + C - 1) / C;
    constexpr bool DECAY = VAR != DELTANET;
    // reverse state pass: value blocks of 32 columns (bf16) when that gives a
    // workgroup per compute unit, else of 16 (twice the sequential chains)
    if (sizeof(E) == 2 && P.dv % 32 == 0 && heads * (P.dv / 32) >= P.cus) {
        const dim3 grid((unsigned)(heads * (P.dv / 32))), block(512);
        hipLaunchKernelGGL((backward_state_kernel<E, DECAY, DK, 32, C>), grid, block, 0, st, P);
    } else {
        const dim3 grid((unsigned)(heads * (P.dv / 16))), block(512);
        hipLaunchKernelGGL((backward_state_kernel<E, DECAY, DK, 16, C>), grid, block, 0, st, P);
    }
    if (hipError_t e = hipGetLastError())
        return e;
    if (nc == 0)
        return hipSuccess;
    constexpr int DVH = sizeof(E) == 2 ? 64 : 32;
    const dim3 grid((unsigned)(heads * nc)), block(512);
    if constexpr (VAR == KDA) {
        if (P.w_f32)
            hipLaunchKernelGGL((backward_chunk_kernel<E, VAR, DK, C, DVH, WS_GAIN>), grid, block,
                               0, st, P);
        else if (P.beta_f32)
            hipLaunchKernelGGL((backward_chunk_kernel<E, VAR, DK, C, DVH, WS_BETA_F32>), grid,
                               block, 0, st, P);
        else
            hipLaunchKernelGGL((backward_chunk_kernel<E, VAR, DK, C, DVH, WS_BETA>), grid, block,
                               0, st, P);
    } else {
        hipLaunchKernelGGL((backward_chunk_kernel<E, VAR, DK, C, DVH, WS_BETA>), grid, block, 0,
                           st, P);
    }
    return hipGetLastError();
}

template <typename E, int VAR>
static hipError_t launch_bwd_v(const BackwardParams &P, hipStream_t st) {
    if (P.dk == 128 && P.chunk == 64) {
        if constexpr (sizeof(E) == 2)
            return launch_bwd_vc<E, VAR, 128, 64>(P, st);
        return hipErrorInvalidValue;
    }
    if (P.dk == 128 && P.chunk == 32) return launch_bwd_vc<E, VAR, 128, 32>(P, st);
    if (P.dk == 64 && P.chunk == 64) return launch_bwd_vc<E, VAR, 64, 64>(P, st);
    if (P.dk == 64 && P.chunk == 32) return launch_bwd_vc<E, VAR, 64, 32>(P, st);
    return hipErrorInvalidValue;
}

template <typename E>
static hipError_t launch_bwd_e(const BackwardParams &P, hipStream_t st) {
    switch (P.variant) {
    case DELTANET: return launch_bwd_v<E, DELTANET>(P, st);
    case GATED_DELTANET: return launch_bwd_v<E, GATED_DELTANET>(P, st);
    case KDA: return launch_bwd_v<E, KDA>(P, st);
    case DIAG_KDN: {
        // the memory part with the gains as write vectors, then the
        // per-channel variance chain
        if (hipError_t e = launch_bwd_v<E, KDA>(P, st))
            return e;
        return launch_diag_chain_e<E>(P, st);
    }
    case ISO_KDN: {
        // the memory part as KDA with the derived write strengths, then the
        // variance chain
        if (hipError_t e = launch_bwd_v<E, KDA>(P, st))
            return e;
        const long bh = (long)P.B * P.H, nc = (P.T + P.chunk - 1) / P.chunk;
        if (nc > 0) {
            const dim3 g1((unsigned)((bh * nc + 3) / 4)), b1(256);
            hipLaunchKernelGGL(iso_chain_map_kernel, g1, b1, 0, st, P);
            if (hipError_t e = hipGetLastError())
                return e;
        }
        hipLaunchKernelGGL(chain_scan_kernel, dim3((unsigned)((bh + 3) / 4)), dim3(256), 0, st,
                           P, 1);
        if (hipError_t e = hipGetLastError())
            return e;
        if (nc > 0) {
            const dim3 g3((unsigned)((bh * nc + 3) / 4)), b3(256);
            hipLaunchKernelGGL((iso_chain_grad_kernel<E>), g3, b3, 0, st, P);
        }
        return hipGetLastError();
    }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_backward(const BackwardParams &P, hipStream_t st) {
    if ((long)P.B * P.H == 0)
        return hipSuccess;
    return P.bf16 ? launch_bwd_e<bf16>(P, st) : launch_bwd_e<float>(P, st);
}

}  // namespace kdn
