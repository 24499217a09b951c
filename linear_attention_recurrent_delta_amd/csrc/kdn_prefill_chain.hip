// kdn_prefill_chain.hip -- sequential state pass of the two-pass chunkwise
// prefill for bf16 operands (gfx950), one wave per 16-column block of S.
//
// What is left after the prep kernel is the inter-chunk recurrence
// ("معماری KDA ...", section "حل مشکل وابستگی علی": provisional errors
// resolved by the causal triangular solve):
//   U = V - K~ S,   E = T U,   O = Q~ S + A_qk E,
//   S <- diag(gamma_C) S + W~^T E.
//
// Layout trick.  v_mfma_f32_16x16x32_bf16 contracts over 32 k-slots: lane l
// feeds k-slots (l>>4)*8 + e (e = 0..7) of its A row and B column, and any
// bijection between k-slots and the contraction index is valid as long as
// A and B use the same one.  The accumulator layout puts rows
// (l>>4)*4 + r (r = 0..3) of a 16-row tile in lane l.  The prep kernel
// therefore stores every record matrix with the contraction index of each
// 32-group g permuted as
//   k(g, q, e) = 32 g + (e < 4 ? 4 q + e : 16 + 4 q + e - 4),   q = l >> 4,
// (kdn_workspace.h), and the B operand of each product -- S over d_k, U and
// E over the chunk's tokens -- is the lane's own accumulator registers of two
// adjacent 16-row tiles, rounded to bf16.  The whole chain runs inside one
// wave: no LDS exchange and no barrier between its three products.
//
// v enters without a transposition: its token rows are loaded as A-operand
// fragments (16-byte row segments) and multiplied by -I, which puts -V in the
// accumulator layout of U exactly; K~ S then accumulates onto it, so the
// chain carries -U and -E, and the permuted records hold -W~^T and -A_qk
// (kdn_workspace.h), which turn them back into the S update and the output.
//
// Workgroup = two waves for one (batch*head, 16*NTJ columns of S):
//   wave 0 (chain): S in registers for the whole sequence; per chunk U, E and
//     the S update, then hands S (as it was at the chunk start) and E to
//     wave 1 through a double-buffered LDS slot;
//   wave 1 (output): O = Q~ S + A_qk E for the chunk, stored to o.
// One barrier per chunk orders the hand-off.  Each wave loads its record
// fragments straight from global memory into registers with buffer
// instructions, the next chunk's as soon as the current chunk's are used, and
// the output wave touches one dword per 128-byte line of the block's share of
// the record (and of its v rows) two chunks ahead, so those loads hit L2.  The value blocks of a head
// are placed on one XCD, which then reads each record from HBM once.
#include "kdn_device.h"
#include "kdn_launch.h"
#include "kdn_workspace.h"

namespace kdn {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer access (byte offsets); offsets at or beyond `bytes` read 0 and
// drop stores (32-bit data format in descriptor word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ bf16x8 frag(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0));
}
__device__ __forceinline__ f32x4 load_f4(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0));
}
// 8 accumulator values (two 16-row tiles, rows 4q..4q+3 of each) as the bf16
// B operand of the permuted k-slots
__device__ __forceinline__ bf16x8 pack8(const f32x4 &lo, const f32x4 &hi) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = static_cast<bf16>(lo[e]);
        r[4 + e] = static_cast<bf16>(hi[e]);
    }
    return r;
}
__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

// SAVE (the forward re-run of the gradient computation): the output wave
// writes S at the start of every chunk to P.states ([batch*head][chunk][d_k]
// [d_v], bf16, as rounded for the chunk's products) instead of computing o;
// S_out is not written.
template <bool DECAY, int DK, int C, int NTJ, bool SAVE>
__global__ __launch_bounds__(128) void prefill_chain_kernel(PrefillParams P) {
    constexpr int NB = C / 16;          // 16-row token blocks of a chunk
    constexpr int NIB = DK / 16;        // 16-row key blocks of S
    constexpr int GK = DK / 32;         // 32-groups over d_k
    constexpr int GC = C / 32;          // 32-groups over the chunk's tokens
    constexpr int NV = 16 * NTJ;        // columns of S per workgroup
    static_assert(GK * 32 == DK && GC * 32 == C && GC >= 1, "tiling");
    constexpr int NSF = GK * NTJ;       // S fragments handed to the output wave
    constexpr int NEF = GC * NTJ;       // E fragments
    __shared__ bf16x8 slot[2][(NSF + NEF) * 64];
    // o moves from the accumulator layout to global memory through LDS:
    // 2-byte LDS writes in the MFMA layout, then 16-byte row accesses (LPR
    // lanes per row, RPI rows per instruction, NVI instructions per chunk).
    constexpr int LPR = NV / 8, RPI = 64 / LPR, NVI = C / RPI;
    constexpr int POB = NV + 8;           // o [token][column], pitch (bf16)
    static_assert(RPI * NVI == C && (POB * 2) % 16 == 0, "o tiles");
    __shared__ __attribute__((aligned(16))) bf16 OB[C * POB];

    const int lane = threadIdx.x & 63;
    const bool chain = threadIdx.x < 64;
    const int q = lane >> 4, n = lane & 15;

    // Workgroup -> (batch*head, value block); dispatch is round-robin over
    // the 8 XCDs, so consecutive ids with the same residue mod 8 share one.
    const int nvb = P.dv / NV;
    const int G = gridDim.x;
    int lid = blockIdx.x;
    if ((G & 7) == 0 && ((G >> 3) % nvb) == 0)
        lid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int bh = lid / nvb, vb = lid % nvb;
    const int b = bh / P.H, h = bh % P.H;
    const int T = P.T, H = P.H, DV = P.dv;
    const int v0 = vb * NV;
    const int NC = (T + C - 1) / C;
    const WsLayout LW = WsLayout::make(1, C, DK);
    const char *ws = static_cast<const char *>(P.ws) + (long)bh * NC * LW.rec;
    const long hdv = (long)H * DV;                         // token stride of v, o
    const long seq0 = ((long)b * T * H + h) * DV + v0;     // (b, t = 0, h, v0)
    const bf16 *gv = static_cast<const bf16 *>(P.v);
    bf16 *go = static_cast<bf16 *>(P.o);
    const unsigned lane16 = (unsigned)lane * 16u;
    // v / o element (t = 16 m + 4 q + r, column 16 j + n) of a chunk: the lane
    // part in a register, the (m, r, j) part as a uniform offset
    // row access of the v / o tiles: lane -> (token row, 8 columns)
    const int rrow = lane / LPR, rcol = (lane % LPR) * 8;
    const unsigned rlane = (unsigned)((rrow * hdv + rcol) * 2);
    auto rsoff = [&](int h) { return (int)(h * RPI * hdv * 2); };
    auto rec = [&](int c) { return rsrc(ws + (long)c * LW.rec, (unsigned)LW.rec); };
    // rows [c C, c C + L) of v or o in range; the rest read 0 / are dropped
    auto rows = [&](const bf16 *base, int c) {
        const int L = min(C, T - c * C);
        return rsrc(base + seq0 + (long)c * C * hdv, (unsigned)(((L - 1) * hdv + NV) * 2));
    };

    if (chain) {
        // S[16 i + 4 q + r][v0 + 16 j + n] in sacc[i][j][r]
        f32x4 sacc[NIB][NTJ];
#pragma unroll
        for (int i = 0; i < NIB; ++i)
#pragma unroll
            for (int j = 0; j < NTJ; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sacc[i][j][r] = P.S0 ? P.S0[((long)bh * DK + 16 * i + 4 * q + r) * DV +
                                                v0 + 16 * j + n]
                                         : 0.f;
        bf16x8 kf[NB][GK], tf[NB][GC], wf[NIB][GC];
        f32x4 gm[NIB];
        // v of the chunk as A-operand fragments: vf[m] holds token row
        // 16 m + n, columns 8 q .. 8 q + 7 of the block (zero for q >= NV / 8),
        // so that -V comes out of one MFMA per tile against -I (below) in the
        // accumulator layout of U, with no transposition
        bf16x8 vf[NB];
        unsigned voff[NB];
        // lanes past the block's columns: an offset at the range of a whole
        // chunk, which no chunk's descriptor reaches
        const unsigned vdead = (unsigned)(((C - 1) * hdv + NV) * 2);
#pragma unroll
        for (int m = 0; m < NB; ++m)
            voff[m] = 8 * q < NV ? (unsigned)(((16 * m + n) * hdv + 8 * q) * 2) : vdead;
        // B operand -I for column tile j: k-slot 8 q + e (column 8 q + e of
        // the block) against column 16 j + n
        bf16x8 nid[NTJ];
#pragma unroll
        for (int j = 0; j < NTJ; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                nid[j][e] = static_cast<bf16>(8 * q + e == 16 * j + n ? -1.f : 0.f);
        auto load_k = [&](int c) {
            const auto rr = rec(c);
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int g = 0; g < GK; ++g)
                    kf[m][g] = frag(rr, lane16, (int)LW.off_kd + (m * GK + g) * 1024);
        };
        // rows past the sequence end and columns past the block read 0
        auto load_v = [&](int c) {
            const auto vrr = rows(gv, c);
#pragma unroll
            for (int m = 0; m < NB; ++m)
                vf[m] = frag(vrr, voff[m], 0);
        };
        auto load_t = [&](int c) {
            const auto rr = rec(c);
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int g = 0; g < GC; ++g)
                    if (32 * g <= 16 * m + 15)   // T is lower triangular
                        tf[m][g] = frag(rr, lane16, (int)LW.off_tm + (m * GC + g) * 1024);
        };
        auto load_w = [&](int c) {
            const auto rr = rec(c);
#pragma unroll
            for (int i = 0; i < NIB; ++i)
#pragma unroll
                for (int g = 0; g < GC; ++g)
                    wf[i][g] = frag(rr, lane16, (int)LW.off_wdt + (i * GC + g) * 1024);
        };
        auto load_g = [&](int c) {
            if (DECAY) {
                const auto rr = rec(c);
#pragma unroll
                for (int i = 0; i < NIB; ++i)
                    gm[i] = load_f4(rr, (unsigned)(q * 16), (int)LW.off_gc + i * 64);
            }
        };
        // Every operand is loaded one chunk before its use, in the order of
        // use, so each wait is for a load issued a chunk period earlier:
        // gamma_C at the chunk start, then K~ and v (U), T (E), W~^T (S).
        if (NC > 0) {
            load_g(0);
            load_k(0);
            load_v(0);
            load_t(0);
            load_w(0);
        }
        for (int c = 0; c < NC; ++c) {
            const int cn = min(c + 1, NC - 1);   // the last chunk reloads itself
            bf16x8 *sl = slot[c & 1];
            // S at the chunk start as the B operand over d_k; handed on
            bf16x8 sb[GK][NTJ];
#pragma unroll
            for (int g = 0; g < GK; ++g)
#pragma unroll
                for (int j = 0; j < NTJ; ++j) {
                    sb[g][j] = pack8(sacc[2 * g][j], sacc[2 * g + 1][j]);
                    sl[(g * NTJ + j) * 64 + lane] = sb[g][j];
                }
            // the decay part of the S update, diag(gamma_C) S, now that the
            // operand copy of S is taken; then the next chunk's gamma_C
            if (DECAY) {
#pragma unroll
                for (int i = 0; i < NIB; ++i)
#pragma unroll
                    for (int j = 0; j < NTJ; ++j)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            sacc[i][j][r] *= gm[i][r];
                load_g(cn);
            }
            // -U = K~ S - V: the accumulators start at -V (V times -I, exact)
            // and K~ S accumulates onto them
            f32x4 ua[NB][NTJ];
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int j = 0; j < NTJ; ++j)
                    ua[m][j] = mfma(vf[m], nid[j], f32x4{0.f, 0.f, 0.f, 0.f});
            load_v(cn);
#pragma unroll
            for (int g = 0; g < GK; ++g)
#pragma unroll
                for (int m = 0; m < NB; ++m)
#pragma unroll
                    for (int j = 0; j < NTJ; ++j)
                        ua[m][j] = mfma(kf[m][g], sb[g][j], ua[m][j]);
            load_k(cn);
            bf16x8 ub[GC][NTJ];
#pragma unroll
            for (int g = 0; g < GC; ++g)
#pragma unroll
                for (int j = 0; j < NTJ; ++j)
                    ub[g][j] = pack8(ua[2 * g][j], ua[2 * g + 1][j]);
            // -E = T (-U) (T lower triangular: groups at or left of the diagonal)
            f32x4 ea[NB][NTJ];
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int j = 0; j < NTJ; ++j) {
                    ea[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int g = 0; g < GC; ++g)
                        if (32 * g <= 16 * m + 15)
                            ea[m][j] = mfma(tf[m][g], ub[g][j], ea[m][j]);
                }
            load_t(cn);
            bf16x8 eb[GC][NTJ];
#pragma unroll
            for (int g = 0; g < GC; ++g)
#pragma unroll
                for (int j = 0; j < NTJ; ++j) {
                    eb[g][j] = pack8(ea[2 * g][j], ea[2 * g + 1][j]);
                    sl[(NSF + g * NTJ + j) * 64 + lane] = eb[g][j];
                }
            __syncthreads();
            // S <- diag(gamma_C) S + W~^T E, as (-W~^T) (-E) from the record
#pragma unroll
            for (int g = 0; g < GC; ++g)
#pragma unroll
                for (int i = 0; i < NIB; ++i)
#pragma unroll
                    for (int j = 0; j < NTJ; ++j)
                        sacc[i][j] = mfma(wf[i][g], eb[g][j], sacc[i][j]);
            load_w(cn);
        }
        if constexpr (!SAVE) {
#pragma unroll
            for (int i = 0; i < NIB; ++i)
#pragma unroll
                for (int j = 0; j < NTJ; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        P.S_out[((long)bh * DK + 16 * i + 4 * q + r) * DV + v0 + 16 * j + n] =
                            sacc[i][j][r];
        }
    } else if constexpr (SAVE) {
        // S of chunk c from the slot into rows of an LDS tile (lane (q, n) of
        // fragment (g, j) holds rows 32 g + 4 q + e (e < 4) and 32 g + 16 +
        // 4 q + e - 4 of column 16 j + n), then 16-byte row segments out
        constexpr int PSB = NV + 8, SPR = NV / 8, NSU = DK * SPR / 64;
        static_assert(NSU * 64 == DK * SPR, "state rows");
        __shared__ __attribute__((aligned(16))) unsigned short SBT[DK * PSB];
        bf16 *gs = static_cast<bf16 *>(P.states) + (long)bh * NC * DK * DV;
        unsigned pf[5];
        auto touch = [&](int cn) {      // as the output wave's L2 probes below
            const bool in = cn < NC;
            const int cc = in ? cn : 0;
            const auto rr = rsrc(ws + (long)cc * LW.rec, in ? (unsigned)LW.rec : 0u);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                pf[k] = __builtin_amdgcn_raw_buffer_load_b32(
                    rr, (int)(((k * 64 + lane) * nvb + vb) * 128), 0, 0);
            const int L = min(C, T - cc * C);
            const auto vrr = rsrc(gv + seq0 + (long)cc * C * hdv,
                                  in ? (unsigned)(((L - 1) * hdv + NV) * 2) : 0u);
            pf[4] = __builtin_amdgcn_raw_buffer_load_b32(vrr, (int)(lane * hdv * 2), 0, 0);
            asm volatile("" ::: "memory");
        };
        if (NC > 0)
            touch(1);
        for (int c = 0; c < NC; ++c) {
            __syncthreads();
            const bf16x8 *sl = slot[c & 1];
#pragma unroll
            for (int g = 0; g < GK; ++g)
#pragma unroll
                for (int j = 0; j < NTJ; ++j) {
                    // (halves taken from the 32-bit words: a bf16 element
                    // extracted from the vector for a 16-bit store compiled
                    // to element 0 every time)
                    const u32x4 x = __builtin_bit_cast(u32x4, sl[(g * NTJ + j) * 64 + lane]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = 32 * g + 4 * q + (e < 4 ? e : 12 + e);
                        const unsigned w = x[e >> 1];
                        SBT[row * PSB + 16 * j + n] =
                            (unsigned short)((e & 1) ? w >> 16 : w & 0xffffu);
                    }
                }
#pragma unroll
            for (int k = 0; k < 5; ++k)
                asm volatile("" ::"v"(pf[k]));
            touch(c + 2);
            const auto srr = rsrc(gs + (long)c * DK * DV, (unsigned)(DK * DV * 2));
#pragma unroll
            for (int u = 0; u < NSU; ++u) {
                const int x = u * 64 + lane, r = x / SPR, hs = x % SPR;
                const u32x4 val = *reinterpret_cast<const u32x4 *>(SBT + r * PSB + 8 * hs);
                __builtin_amdgcn_raw_buffer_store_b128(val, srr, (r * DV + v0 + 8 * hs) * 2, 0, 0);
            }
        }
        if (NC > 0) {
#pragma unroll
            for (int k = 0; k < 5; ++k)
                asm volatile("" ::"v"(pf[k]));
        }
    } else {
        bf16x8 qf[NB][GK], af[NB][GC];
        auto load_qa = [&](int c) {
            const auto rr = rec(c);
#pragma unroll
            for (int m = 0; m < NB; ++m) {
#pragma unroll
                for (int g = 0; g < GK; ++g)
                    qf[m][g] = frag(rr, lane16, (int)LW.off_qd + (m * GK + g) * 1024);
#pragma unroll
                for (int g = 0; g < GC; ++g)
                    if (32 * g <= 16 * m + 15)
                        af[m][g] = frag(rr, lane16, (int)LW.off_aqk + (m * GC + g) * 1024);
            }
        };
        unsigned pf[5];
        // one dword of each 128-byte line of this block's share of chunk cn's
        // record, and of its v rows; chunks past the end read through an
        // empty descriptor (no memory touched)
        auto touch = [&](int cn) {
            // descriptor fields selected as scalars, so no branch (and no
            // path-dependent wait count) is generated
            const bool in = cn < NC;
            const int cc = in ? cn : 0;
            const auto rr = rsrc(ws + (long)cc * LW.rec, in ? (unsigned)LW.rec : 0u);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                pf[k] = __builtin_amdgcn_raw_buffer_load_b32(
                    rr, (int)(((k * 64 + lane) * nvb + vb) * 128), 0, 0);
            const int L = min(C, T - cc * C);
            const auto vrr = rsrc(gv + seq0 + (long)cc * C * hdv,
                                  in ? (unsigned)(((L - 1) * hdv + NV) * 2) : 0u);
            pf[4] = __builtin_amdgcn_raw_buffer_load_b32(vrr, (int)(lane * hdv * 2), 0, 0);
            asm volatile("" ::: "memory");
        };
        if (NC > 0) {
            load_qa(0);
            touch(1);
        }
        for (int c = 0; c < NC; ++c) {
            const int cn = min(c + 1, NC - 1);
            __syncthreads();
            const bf16x8 *sl = slot[c & 1];
            bf16x8 sb[GK][NTJ], eb[GC][NTJ];
#pragma unroll
            for (int g = 0; g < GK; ++g)
#pragma unroll
                for (int j = 0; j < NTJ; ++j)
                    sb[g][j] = sl[(g * NTJ + j) * 64 + lane];
#pragma unroll
            for (int g = 0; g < GC; ++g)
#pragma unroll
                for (int j = 0; j < NTJ; ++j)
                    eb[g][j] = sl[(NSF + g * NTJ + j) * 64 + lane];
            f32x4 oa[NB][NTJ];
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int j = 0; j < NTJ; ++j)
                    oa[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int g = 0; g < GK; ++g)
#pragma unroll
                for (int m = 0; m < NB; ++m)
#pragma unroll
                    for (int j = 0; j < NTJ; ++j)
                        oa[m][j] = mfma(qf[m][g], sb[g][j], oa[m][j]);
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int g = 0; g < GC; ++g)
                    if (32 * g <= 16 * m + 15)
#pragma unroll
                        for (int j = 0; j < NTJ; ++j)
                            oa[m][j] = mfma(af[m][g], eb[g][j], oa[m][j]);
            // the previous chunk's L2 probes are retired here, after this
            // chunk's operands, which were issued after them
#pragma unroll
            for (int k = 0; k < 5; ++k)
                asm volatile("" ::"v"(pf[k]));
            load_qa(cn);
            touch(c + 2);
            // o through LDS into rows: 2-byte writes in the MFMA layout, then
            // 16-byte reads and stores of whole row segments (rows past the
            // sequence end fall outside the descriptor and are dropped)
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < NTJ; ++j)
                        OB[(16 * m + 4 * q + r) * POB + 16 * j + n] =
                            static_cast<bf16>(oa[m][j][r]);
            const auto orr = rows(go, c);
#pragma unroll
            for (int h = 0; h < NVI; ++h) {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(OB + (h * RPI + rrow) * POB + rcol);
                __builtin_amdgcn_raw_buffer_store_b128(x, orr, (int)rlane, rsoff(h), 0);
            }
        }
        if (NC > 0) {
#pragma unroll
            for (int k = 0; k < 5; ++k)
                asm volatile("" ::"v"(pf[k]));
        }
    }
}

template <bool DECAY, int DK, int C, int NTJ>
static hipError_t launch_chain_one(const PrefillParams &P, hipStream_t st) {
    const long heads = (long)P.B * P.H;
    const dim3 grid((unsigned)(heads * (P.dv / (16 * NTJ)))), block(128);
    if (P.states)
        hipLaunchKernelGGL((prefill_chain_kernel<DECAY, DK, C, NTJ, true>), grid, block, 0, st, P);
    else
        hipLaunchKernelGGL((prefill_chain_kernel<DECAY, DK, C, NTJ, false>), grid, block, 0, st, P);
    return hipGetLastError();
}

#ifndef KDN_CHAIN_NTJ
#define KDN_CHAIN_NTJ 0
#endif

// Column tiles per chain wave: one (16 columns) while that gives at least one
// workgroup per CU, else two.
static int chain_tiles(const PrefillParams &P) {
    if (KDN_CHAIN_NTJ)
        return KDN_CHAIN_NTJ;
    const long heads = (long)P.B * P.H;
    return (P.dv % 32 == 0 && heads * (P.dv / 32) >= P.cus) ? 2 : 1;
}

template <bool DECAY, int DK, int C>
static hipError_t launch_chain_c(const PrefillParams &P, hipStream_t st) {
    return chain_tiles(P) == 2 ? launch_chain_one<DECAY, DK, C, 2>(P, st)
                               : launch_chain_one<DECAY, DK, C, 1>(P, st);
}

template <bool DECAY, int DK>
static hipError_t launch_chain_dk(const PrefillParams &P, hipStream_t st) {
    if (P.chunk == 64) return launch_chain_c<DECAY, DK, 64>(P, st);
    if (P.chunk == 32) return launch_chain_c<DECAY, DK, 32>(P, st);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_chain(const PrefillParams &P, hipStream_t st) {
    if (!P.bf16 || !P.rec_perm)
        return hipErrorInvalidValue;
    const bool decay = P.variant != DELTANET;
    if (P.dk == 128)
        return decay ? launch_chain_dk<true, 128>(P, st) : launch_chain_dk<false, 128>(P, st);
    if (P.dk == 64)
        return decay ? launch_chain_dk<true, 64>(P, st) : launch_chain_dk<false, 64>(P, st);
    return hipErrorInvalidValue;
}

}  // namespace kdn
