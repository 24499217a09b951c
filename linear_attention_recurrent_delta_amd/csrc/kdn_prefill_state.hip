// kdn_prefill_state.hip -- sequential state pass of the two-pass chunkwise
// prefill on gfx950.
//
// The prep kernel has already written, per chunk, the S-independent
// quantities K~, Q~, W~^T, A_qk, T and gamma_C (kdn_workspace.h).  What is
// left is the inter-chunk recurrence ("معماری KDA ...", section "حل مشکل
// وابستگی علی": provisional errors resolved by the causal triangular solve):
//   U = V - K~ S,   E = T U,   O = Q~ S + A_qk E,   S <- diag(gamma_C) S + W~^T E.
//
// One workgroup of eight waves owns one (batch*head, NV-column block of S).
// S stays in registers in MFMA accumulator layout for the whole sequence and
// is mirrored in LDS (operand type, [col][row]) for the products that read
// it.  Waves 0-3 carry the serial chain of token block w (U = V - K~ S, then
// E = T U); waves 4-7 the output of token block w-4 (Q~ S while the chain
// runs, A_qk E one chunk later from a second E^T buffer); every wave updates
// its S tiles.  Every A operand (the prep kernel's matrices) is loaded
// straight from global memory into registers in fragment order, one chunk
// ahead, and the record two chunks ahead is prefetched into L2, so the only
// LDS traffic is the S / U / E exchange between the MFMA output and operand
// layouts.  Three barriers per chunk.
//
// SAVE (the forward pass of a float32 gradient computation; bf16 ones use the
// chain kernel's SAVE mode): S at the start of every chunk is written to
// P.states ([batch*head][chunk][d_k][d_v], float32), and neither o nor S_out
// is written.
#include "kdn_device.h"
#include "kdn_launch.h"
#include "kdn_workspace.h"


namespace kdn {

// Distance in chunks from the chunk whose operands a wave loads to the chunk
// it prefetches into L2 at the same time (0: no prefetch).
#ifndef KDN_STATE_PFD
#define KDN_STATE_PFD 2
#endif

typedef uint4 Frag;   // 16 bytes of an A-operand fragment

template <typename E> struct FragMma;

// acc += A(16 x 32) * B(32 x 16): A from a bf16 fragment, B from LDS as
// [col][k] (pitch ldb, k offset k0).
template <> struct FragMma<bf16> {
    static constexpr int KG = 32;
    __device__ __forceinline__ static void mma(f32x4 &acc, const Frag &a, const bf16 *B,
                                               int ldb, int k0, int lane) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, a);
        const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(
            B + (lane & 15) * ldb + k0 + (lane >> 4) * 8);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
};

// acc += A(16 x 16) * B(16 x 16) as four fp32 MFMA steps of k = 4.
template <> struct FragMma<float> {
    static constexpr int KG = 16;
    __device__ __forceinline__ static void mma(f32x4 &acc, const Frag &a, const float *B,
                                               int ldb, int k0, int lane) {
        const float4 af = __builtin_bit_cast(float4, a);
        const float *pb = B + (lane & 15) * ldb + k0 + (lane >> 4);
        const float b0 = pb[0], b1 = pb[4], b2 = pb[8], b3 = pb[12];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af.x, b0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af.y, b1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af.z, b2, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af.w, b3, acc, 0, 0, 0);
    }
};

// Raw buffer access (offsets in bytes).  Word 3 of the descriptor selects
// 32-bit data format so the range check applies; offsets at or beyond
// `bytes` read as 0 and drop stores.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ Frag buf_frag(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
    return __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0));
}
// One element as raw bits in a 32-bit register (bf16: the low half), and its
// value.  Kept as 32-bit words, separate loads are never packed into one
// register, which would make the wave wait for them at once.
template <typename E> __device__ __forceinline__ unsigned buf_raw(__amdgpu_buffer_rsrc_t r, unsigned voff);
template <> __device__ __forceinline__ unsigned buf_raw<bf16>(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return (unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, 0, 0);
}
template <> __device__ __forceinline__ unsigned buf_raw<float>(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
}
template <typename E> __device__ __forceinline__ float raw_f32(unsigned x) {
    return __builtin_bit_cast(float, sizeof(E) == 2 ? x << 16 : x);
}
template <typename E> __device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, unsigned voff, E x);
template <> __device__ __forceinline__ void buf_store<bf16>(__amdgpu_buffer_rsrc_t r, unsigned voff, bf16 x) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, (int)voff, 0, 0);
}
template <> __device__ __forceinline__ void buf_store<float>(__amdgpu_buffer_rsrc_t r, unsigned voff, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, (int)voff, 0, 0);
}

template <typename E, bool DECAY, int DK, int NV, int C, bool SAVE>
__global__ __launch_bounds__(512) void prefill_state_kernel(PrefillParams P) {
    constexpr int KG = FragMma<E>::KG;
    constexpr int NB = C / 16;          // token blocks of a chunk
    constexpr int NTJ = NV / 16;        // column tiles of the S block
    constexpr int NIBT = DK / 16;       // key blocks of S
    constexpr int NSTT = NIBT * NTJ;    // S tiles
    constexpr int NSW = (NSTT + 7) / 8; // S tiles per wave (max)
    constexpr int GK = DK / KG;         // fragment groups over DK
    constexpr int GC = C / KG;          // fragment groups over C
    constexpr int PADE = 16 / (int)sizeof(E);
    constexpr int PK = DK + PADE, PC = C + PADE;
    static_assert(GK * KG == DK && GC * KG == C && NB <= 4, "tiling");
    static_assert(8 % NIBT == 0 || NIBT % 8 == 0, "S tiles of a wave share one key block");

    __shared__ __attribute__((aligned(16))) E ST[NV * PK];   // S^T block
    __shared__ __attribute__((aligned(16))) E UT[NV * PC];   // U^T
    __shared__ __attribute__((aligned(16))) E ETB[2][NV * PC]; // E^T, by chunk parity

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // waves 0-3: the serial chain U -> E for token block wv;
    // waves 4-7: the output path of token block wv - 4;
    // all waves: S tiles tau = wv + 8k, (key block, column tile) =
    //            (tau % NIBT, tau / NIBT).
    const bool chain = wv < NB;
    const bool outw = wv >= 4 && wv - 4 < NB;
    const int m = chain ? wv : wv - 4;          // token block
    const int ib = wv % NIBT;                   // key block of this wave's S tiles

    // Workgroup -> (batch*head, value block); the value blocks of one head
    // land on one XCD (dispatch is round-robin over the 8 XCDs), so they
    // share the head's workspace records through that XCD's L2.
    const int nvb = P.dv / NV;
    const int G = gridDim.x;
    const bool remap = (G & 7) == 0 && ((G >> 3) % nvb) == 0;
    int lid = blockIdx.x;
    if (remap)
        lid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int bh = lid / nvb, vb = lid % nvb;
    const int b = bh / P.H, h = bh % P.H;
    const int v0 = vb * NV;
    const int T = P.T, H = P.H, DV = P.dv;
    const int NC = (T + C - 1) / C;     // chunks
    const WsLayout LW = WsLayout::make(sizeof(E) == 2, C, DK);
    const char *ws = static_cast<const char *>(P.ws) + (long)bh * NC * LW.rec;
    const E *gv = static_cast<const E *>(P.v);
    E *go = static_cast<E *>(P.o);

    // S tiles in accumulator layout: sacc[k][r] =
    //   S[ib*16 + (lane>>4)*4 + r][v0 + nj_k*16 + (lane&15)],  nj_k = (wv + 8k) / NIBT
    f32x4 sacc[NSW];
    const int i0 = ib * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int k = 0; k < NSW; ++k) {
        const int tau = wv + 8 * k;
        if (tau >= NSTT) continue;
        const int j = (tau / NIBT) * 16 + (lane & 15);
        float s4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sacc[k][r] = P.S0 ? P.S0[((long)bh * DK + i0 + r) * DV + v0 + j] : 0.f;
            s4[r] = sacc[k][r];
        }
        lds_stn<4>(ST + j * PK + i0, s4);
    }

    // One chunk's operands for this wave: the token-block fragments (K~ and T
    // for a chain wave, Q~ and A_qk for an output wave), the W~^T key block
    // and gamma_C of its S tiles, and (chain waves) the v tile.
    constexpr int REC = (int)WsLayout::make(sizeof(E) == 2, C, DK).rec;
    constexpr int NPF = (REC + 512 * 128 - 1) / (512 * 128);
    struct Chunk {
        Frag kq[GK], ta[GC], wt[GC], gc;
        unsigned v[NTJ][4];             // raw bits of the v tile
        unsigned pf[NPF + 1];           // L2 prefetch probes (see touch)
    };
    // Memory access: buffer instructions with a wave-uniform descriptor per
    // chunk (scalar registers) and per-lane byte offsets fixed for the whole
    // sequence, so no vector address arithmetic runs per chunk.  Rows of v
    // and o past the end of the sequence fall outside the descriptor's range:
    // those loads return 0 and those stores are dropped by the hardware.
    const unsigned lane16 = (unsigned)lane * 16u;          // fragment slot
    const long hdv = (long)H * DV;                         // token stride of v, o
    const long seq0 = ((long)b * T * H + h) * DV + v0;     // (b, t=0, h, v0)
    unsigned vofs[NTJ][4];                                 // byte offsets in a chunk
#pragma unroll
    for (int nj = 0; nj < NTJ; ++nj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            vofs[nj][r] = (unsigned)(((m * 16 + (lane >> 4) * 4 + r) * hdv +
                                      (lane & 15) + nj * 16) * (long)sizeof(E));
    const unsigned gc_lane = (unsigned)(lane >> 4) * 16u;
    const int okq = (int)(chain ? LW.off_kd : LW.off_qd) + m * GK * 1024;
    const int ota = (int)(chain ? LW.off_tm : LW.off_aqk) + m * GC * 1024;
    const int owt = (int)LW.off_wdt + ib * GC * 1024;
    const int ogc = (int)LW.off_gc + ib * 64;
    auto rec_rsrc = [&](int c) { return buf_rsrc(ws + (long)c * LW.rec, (unsigned)LW.rec); };
    // v / o rows of chunk c: [c*C, c*C + L) in range
    auto row_rsrc = [&](const E *base, int c) {
        const int L = min(C, T - c * C);
        return buf_rsrc(base + seq0 + (long)c * C * hdv,
                        (unsigned)(((L - 1) * hdv + NV) * (long)sizeof(E)));
    };

    // L2 prefetch of chunk cn into X.pf: one dword of every 128-byte line of
    // its record (read by one value block of the head when the head's blocks
    // share an XCD, by every block otherwise) and, wave 0, of this block's v
    // rows.  Each dword has a register of its own that nothing reads until
    // the end of the chunk computed from X (an empty asm statement uses it
    // there), so the wave waits for these loads no earlier than for the next
    // chunk's operands, issued after them.  Chunks past the end, and the v
    // rows in waves other than 0, read through an empty descriptor, which
    // touches no memory.
    auto touch = [&](Chunk &X, int cn) {
        const bool mine = !remap || vb == cn % nvb;
        const auto rr = (cn < NC && mine) ? rec_rsrc(cn) : buf_rsrc(ws, 0u);
#pragma unroll
        for (int i = 0; i < NPF; ++i)
            X.pf[i] = __builtin_amdgcn_raw_buffer_load_b32(rr, (tid + i * 512) * 128, 0, 0);
        const auto vr = (cn < NC && wv == 0) ? row_rsrc(gv, cn) : buf_rsrc(gv, 0u);
        X.pf[NPF] = __builtin_amdgcn_raw_buffer_load_b32(vr, (unsigned)(lane * hdv * (long)sizeof(E)), 0, 0);
        asm volatile("" ::: "memory");   // keeps the loads here, ahead of the compute
    };
    auto load = [&](Chunk &X, int c) {
        const auto rr = rec_rsrc(c);
        if (chain || outw) {
#pragma unroll
            for (int g = 0; g < GK; ++g)
                X.kq[g] = buf_frag(rr, lane16, okq + g * 1024);
#pragma unroll
            for (int g = 0; g < GC; ++g)
                X.ta[g] = buf_frag(rr, lane16, ota + g * 1024);
        }
        if (wv < NSTT) {
#pragma unroll
            for (int g = 0; g < GC; ++g)
                X.wt[g] = buf_frag(rr, lane16, owt + g * 1024);
            if (DECAY)
                X.gc = buf_frag(rr, gc_lane, ogc);
        }
        if (chain) {
            const auto vr = row_rsrc(gv, c);
#pragma unroll
            for (int nj = 0; nj < NTJ; ++nj)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    X.v[nj][r] = buf_raw<E>(vr, vofs[nj][r]);
        }
        // issued after the operands, so waiting for those does not wait for it
        if (KDN_STATE_PFD > 0)
            touch(X, c + KDN_STATE_PFD);
    };

    // Output waves: Q~ S of chunk c in phase 1, finished in phase 2 of chunk
    // c+1 with A_qk E (E^T of chunk c is kept in the other E^T buffer).
    f32x4 accq[NTJ], accn[NTJ];
    Frag aq_prev[GC];
#pragma unroll
    for (int nj = 0; nj < NTJ; ++nj)
        accq[nj] = accn[nj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < GC; ++g)
        aq_prev[g] = Frag{0u, 0u, 0u, 0u};
    // c = -1 (before the first chunk) stores through an empty descriptor:
    // every store is dropped, and no branch guards it.
    auto finish_output = [&](int c) {
        const auto orr = (!SAVE && c >= 0) ? row_rsrc(go, c) : buf_rsrc(go, 0u);
        const E *ET = ETB[c & 1];
#pragma unroll
        for (int nj = 0; nj < NTJ; ++nj) {
#pragma unroll
            for (int g = 0; g < GC; ++g)
                if (g * KG < (m + 1) * 16)
                    FragMma<E>::mma(accq[nj], aq_prev[g], ET + nj * 16 * PC, PC, g * KG, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                buf_store<E>(orr, vofs[nj][r], from_f32<E>(accq[nj][r]));
        }
    };

    auto compute = [&](const Chunk &X, int c) {
        if constexpr (SAVE) {
            E *sv = static_cast<E *>(P.states) + ((long)bh * NC + c) * DK * DV;
#pragma unroll
            for (int k = 0; k < NSW; ++k) {
                const int tau = wv + 8 * k;
                if (NSTT % 8 != 0 && tau >= NSTT) continue;
                const int j = (tau / NIBT) * 16 + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sv[(long)(i0 + r) * DV + v0 + j] = from_f32<E>(sacc[k][r]);
            }
        }
        // phase 1: chain waves U = V - K~ S; output waves finish chunk c-1
        // and start Q~ S of chunk c
        if (chain) {
#pragma unroll
            for (int nj = 0; nj < NTJ; ++nj) {
                f32x4 accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < GK; ++g)
                    FragMma<E>::mma(accu, X.kq[g], ST + nj * 16 * PK, PK, g * KG, lane);
                float u[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    u[r] = raw_f32<E>(X.v[nj][r]) - accu[r];
                lds_stn<4>(UT + (nj * 16 + (lane & 15)) * PC + m * 16 + (lane >> 4) * 4, u);
            }
        } else if (outw) {
#pragma unroll
            for (int nj = 0; nj < NTJ; ++nj) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < GK; ++g)
                    FragMma<E>::mma(a, X.kq[g], ST + nj * 16 * PK, PK, g * KG, lane);
                accn[nj] = a;
            }
        }
        __syncthreads();
        E *ET = ETB[c & 1];
        // phase 2: E = T U (chain waves); output waves finish chunk c-1
        if (outw) {
            finish_output(c - 1);
#pragma unroll
            for (int nj = 0; nj < NTJ; ++nj)
                accq[nj] = accn[nj];
#pragma unroll
            for (int g = 0; g < GC; ++g)
                aq_prev[g] = X.ta[g];
        }
        if (chain) {
#pragma unroll
            for (int nj = 0; nj < NTJ; ++nj) {
                f32x4 acce = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < GC; ++g)
                    if (g * KG < (m + 1) * 16)
                        FragMma<E>::mma(acce, X.ta[g], UT + nj * 16 * PC, PC, g * KG, lane);
                float e[4] = {acce[0], acce[1], acce[2], acce[3]};
                lds_stn<4>(ET + (nj * 16 + (lane & 15)) * PC + m * 16 + (lane >> 4) * 4, e);
            }
        }
        __syncthreads();
        // phase 3: S <- diag(gamma_C) S + W~^T E (all waves)
        const float4 g4 = __builtin_bit_cast(float4, X.gc);
#pragma unroll
        for (int k = 0; k < NSW; ++k) {
            const int tau = wv + 8 * k;
            if (NSTT % 8 != 0 && tau >= NSTT) continue;
            const int nj = tau / NIBT;
            if (DECAY) {
                sacc[k][0] *= g4.x;
                sacc[k][1] *= g4.y;
                sacc[k][2] *= g4.z;
                sacc[k][3] *= g4.w;
            }
#pragma unroll
            for (int g = 0; g < GC; ++g)
                FragMma<E>::mma(sacc[k], X.wt[g], ET + nj * 16 * PC, PC, g * KG, lane);
            float s4[4] = {sacc[k][0], sacc[k][1], sacc[k][2], sacc[k][3]};
            lds_stn<4>(ST + (nj * 16 + (lane & 15)) * PK + i0, s4);
        }
        __syncthreads();
        if (KDN_STATE_PFD > 0) {
#pragma unroll
            for (int i = 0; i <= NPF; ++i)
                asm volatile("" ::"v"(X.pf[i]));
        }
    };

    // Software pipeline: chunk c+1's operands load while chunk c computes
    // (the last chunk re-loads itself rather than branching around a load).
    __syncthreads();
    Chunk A, B;
    if (NC > 0)
        load(A, 0);
    for (int c = 0; c < NC; c += 2) {
        load(B, min(c + 1, NC - 1));
        compute(A, c);
        if (c + 1 >= NC)
            break;
        load(A, min(c + 2, NC - 1));
        compute(B, c + 1);
    }
    if (outw && NC > 0)
        finish_output(NC - 1);
    if constexpr (SAVE)
        return;

#pragma unroll
    for (int k = 0; k < NSW; ++k) {
        const int tau = wv + 8 * k;
        if (tau >= NSTT) continue;
        const int j = (tau / NIBT) * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            P.S_out[((long)bh * DK + i0 + r) * DV + v0 + j] = sacc[k][r];
    }
}

template <typename E, bool DECAY, int DK, int NV, int C>
static hipError_t launch_state_one(const PrefillParams &P, hipStream_t st) {
    const long heads = (long)P.B * P.H;
    const dim3 grid((unsigned)(heads * (P.dv / NV))), block(512);
    if (P.states)
        hipLaunchKernelGGL((prefill_state_kernel<E, DECAY, DK, NV, C, true>), grid, block, 0,
                           st, P);
    else
        hipLaunchKernelGGL((prefill_state_kernel<E, DECAY, DK, NV, C, false>), grid, block, 0,
                           st, P);
    return hipGetLastError();
}

#ifndef KDN_STATE_NV
#define KDN_STATE_NV 0
#endif

// Columns of S per workgroup.  Every value block of a head reads the same
// per-chunk operands, so wider blocks cut that traffic; narrower ones give
// more workgroups to fill the CUs.
static int state_value_block(const PrefillParams &P) {
    if (KDN_STATE_NV)
        return KDN_STATE_NV;
    const long heads = (long)P.B * P.H;
    return (P.bf16 && P.dv % 32 == 0 && heads * (P.dv / 32) >= P.cus) ? 32 : 16;
}

template <typename E, bool DECAY, int DK, int C>
static hipError_t launch_state_nv(const PrefillParams &P, hipStream_t st) {
    const int nv = state_value_block(P);
    if (nv == 16) return launch_state_one<E, DECAY, DK, 16, C>(P, st);
    if constexpr (sizeof(E) == 2) {
        if (nv == 32 && P.dv % 32 == 0) return launch_state_one<E, DECAY, DK, 32, C>(P, st);
    }
    return launch_state_one<E, DECAY, DK, 16, C>(P, st);
}

template <typename E, bool DECAY, int DK>
static hipError_t launch_state_c(const PrefillParams &P, hipStream_t st) {
    if (P.chunk == 64) return launch_state_nv<E, DECAY, DK, 64>(P, st);
    if (P.chunk == 32) return launch_state_nv<E, DECAY, DK, 32>(P, st);
    return hipErrorInvalidValue;
}

template <typename E>
static hipError_t launch_state_e(const PrefillParams &P, hipStream_t st) {
    const bool decay = P.variant != DELTANET;
    if (P.dk == 128)
        return decay ? launch_state_c<E, true, 128>(P, st) : launch_state_c<E, false, 128>(P, st);
    if (P.dk == 64)
        return decay ? launch_state_c<E, true, 64>(P, st) : launch_state_c<E, false, 64>(P, st);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_state(const PrefillParams &P, hipStream_t st) {
    return P.bf16 ? launch_state_e<bf16>(P, st) : launch_state_e<float>(P, st);
}

}  // namespace kdn
