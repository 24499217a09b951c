// kdn_workspace.h -- layout of the prefill workspace that carries one chunk's
// S-independent quantities from the chunk-parallel prep kernel to the
// sequential state kernel.
//
// One record per (batch*head, chunk), records ordered [bh][chunk]:
//   Kd   C  x DK   decay-scaled keys     K~ = gamma (.) K
//   Qd   C  x DK   decay-scaled queries  Q~ = gamma (.) Q
//   WdT  DK x C    W~^T, W~_s = (gamma_C / gamma_s) (.) w_s
//   Aqk  C  x C    A_qk (lower triangle, diagonal included)
//   Tm   C  x C    T = (I + A_kk)^-1 (unit lower triangular)
//   gC   DK        gamma_C (float32)
// (chunk algebra: "معماری KDA ...", section "حل مشکل وابستگی علی").
//
// The five matrices are in the operand type E and stored in MFMA A-operand
// fragment order, so that a wave loads the 16-row block it multiplies with
// one coalesced 16-byte load per lane per group:
//   a matrix X[R][K] is cut into 16-row blocks m and k groups g of
//   KG = 16 / sizeof(E) * KSTEP / KPL elements (32 for bf16, 16 for float);
//   lane l of group (m, g) holds 16 bytes at ((m * (K / KG) + g) * 64 + l),
//     bf16 : X[m*16 + (l & 15)][g*32 + (l >> 4)*8 + e],      e = 0..7
//     float: X[m*16 + (l & 15)][g*16 + s*4 + (l >> 4)],       s = 0..3
//   i.e. exactly the A operand of v_mfma_f32_16x16x32_bf16 (one step) or of
//   four v_mfma_f32_16x16x4_f32 steps.
// Permuted order (bf16 only; the forward prefill's records): element e of
// lane l in group g holds column
//     g*32 + (e < 4 ? 4 (l >> 4) + e : 16 + 4 (l >> 4) + e - 4)
//   instead of g*32 + (l >> 4)*8 + e: the k-slots of lane l then line up
//   with the rows 4 (l >> 4) .. + 3 that lane l holds of two adjacent 16-row
//   accumulator tiles, so a product's B operand can be taken from the lane's
//   own accumulators (kdn_prefill_chain.hip).  Permuted records also hold
//   WdT and Aqk negated (-W~^T, -A_qk): the chain kernel carries -U and -E.
__host__ __device__ inline int perm_col(int g, int q, int e) {
    return g * 32 + (e & 4 ? 16 : 0) + 4 * q + (e & 3);
}
//
// For diagonal KDN the workspace also holds, after the records:
//   Mob  [bh][chunk][DK][4] float32  per-chunk composition of the variance
//                                    maps (Mobius form, kdn_variance.hip)
//   P0   [bh][chunk][DK]    float32  variance at each chunk start
//   Pre  [bh][chunk][NS-1][DK][4] float32  maps from the chunk start to the
//                                    start of token segment s = 1 .. NS-1
//                                    (NS = var_segments(DK) segments of C / NS
//                                    tokens), so that the prep kernel runs
//                                    the per-token variance chain of every
//                                    segment at once; within a [DK] block
//                                    channel i sits at pre_pos(i, n, DK),
//                                    n = 16 / element size (the channels one
//                                    lane of the writing kernel holds), so
//                                    that its lanes store contiguous entries
// and for isotropic KDN (one variance per head):
//   Mob  [bh][chunk][4]     float32
//   Stat [bh][chunk][C][4]  float32  per token: mean a^2, mean xi, |k|^2, r
//   P0   [bh][chunk]        float32
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kdn {

struct WsLayout {
    long es;          // bytes per operand element
    int C, DK;
    long off_kd, off_qd, off_wdt, off_aqk, off_tm, off_gc, rec;

    __host__ __device__ static constexpr WsLayout make(int bf16, int C, int DK) {
        WsLayout w{};
        w.es = bf16 ? 2 : 4;
        w.C = C;
        w.DK = DK;
        const long ck = (long)C * DK * w.es, cc = (long)C * C * w.es;
        w.off_kd = 0;
        w.off_qd = w.off_kd + ck;
        w.off_wdt = w.off_qd + ck;
        w.off_aqk = w.off_wdt + ck;
        w.off_tm = w.off_aqk + cc;
        w.off_gc = w.off_tm + cc;
        w.rec = (w.off_gc + (long)DK * 4 + 255) / 256 * 256;
        return w;
    }
    // bytes of the records, and of the whole workspace
    __host__ __device__ long records(long bh, long nc) const { return bh * nc * rec; }
    __host__ __device__ static long mobius_bytes(long bh, long nc, int DK) { return bh * nc * DK * 4 * 4; }
    __host__ __device__ static long p0_bytes(long bh, long nc, int DK) { return bh * nc * DK * 4; }
    __host__ __device__ static long pre_bytes(long bh, long nc, int DK) {
        return bh * nc * (var_segments(DK) - 1) * DK * 4 * 4;
    }
    // Token segments per chunk of the diagonal-KDN variance chain: one thread
    // per (segment, key channel) in the prep kernel's 512 threads.
    __host__ __device__ static constexpr int var_segments(int DK) { return 512 / DK; }
    __host__ __device__ static long stat_bytes(long bh, long nc, int C) { return bh * nc * C * 16; }
};

// Position of key channel i in a [DK] block of segment maps whose writer
// holds n consecutive channels per lane (see Pre above).
__host__ __device__ inline int pre_pos(int i, int n, int DK) { return (i % n) * (DK / n) + i / n; }

// Number of chunks of a sequence of T tokens.
__host__ __device__ inline long num_chunks(long T, int C) { return (T + C - 1) / C; }

}  // namespace kdn
