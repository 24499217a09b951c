// kdn_launch.h -- host-side launch parameters and launchers of the gfx950
// kernels.  The C ABI (kdn_abi.cpp) validates arguments and fills these.
#pragma once

#include <hip/hip_runtime.h>

#include "kdn.h"

namespace kdn {

struct DecodeParams {
    int variant;       // kdn_variant
    int bf16;          // 1: per-token tensors are bfloat16, 0: float32
    int N, H, dk, dv;
    int T;             // tokens per (sequence, head): 1 for a decode step
    float mu;
    const void *q, *k, *v, *alpha, *beta, *xi, *r;   // [N, T, H, .]
    const float *S0;   // [N, H, dk, dv] state read (NULL: zeros); may equal S
    const float *p0;   // [N, H, dk] (diagonal KDN) or [N, H] (isotropic KDN)
                       // variance read; may equal p
    float *S;          // [N, H, dk, dv] state written
    float *p;          // variance written, shaped as p0
    void *o;           // [N, T, H, dv]
};

struct PrefillParams {
    int variant;
    int bf16;
    int B, T, H, dk, dv;
    int chunk;         // C
    float mu;
    const void *q, *k, *v, *alpha, *beta, *xi, *r;
    const float *S0;   // may be null
    const float *p0;   // diagonal KDN
    void *o;
    float *S_out;
    float *p_out;      // diagonal KDN
    // Two-pass schedule (null: single pass).  ws holds the per-chunk records
    // (kdn_workspace.h); ws_mob / ws_p0 the KDN variance scan; ws_pre the
    // diagonal-KDN maps from each chunk start to its token segments; ws_stat
    // the isotropic-KDN per-token sums (mean a^2, mean xi, |k|^2, r).
    void *ws;
    float *ws_mob;
    float *ws_p0;
    float *ws_pre;
    float *ws_stat;
    // Record matrices with the contraction index of each 32-group permuted
    // (kdn_workspace.h), the layout the bf16 chain kernel reads; 0: plain
    // fragment order (the state kernel and the gradient kernels).
    int rec_perm;
    // Gradient computation: S at every chunk start is saved here by the state
    // pass ([batch*head][chunk][dk][dv] in the call's element type, the
    // precision the gradient products read it in; null otherwise).
    void *states;
    // Isotropic KDN, gradient computation: the derived write strengths
    // [B, T, H] (float32) are saved here by the prep kernel (null otherwise).
    float *beta_out;
    // Diagonal KDN, gradient computation: the gains w [B, T, H, dk] and the
    // reciprocal innovation variances 1/s [B, T, H] (0 where s = 0), float32.
    float *w_out;
    float *invs_out;
    int cus;           // compute units of the current device
};

// Gradients of the chunkwise prefill (write-strength variants).  All gradient
// outputs are float32.
struct BackwardParams {
    int variant;
    int bf16;
    int B, T, H, dk, dv;
    int chunk;
    float mu;
    const void *q, *k, *v, *alpha, *beta;   // [B, T, H, .] in the call's dtype
    const void *xi, *r;                     // isotropic KDN: process / observation noise
    const float *p0;                        // isotropic KDN: [B, H]
    const float *beta_f32;                  // isotropic KDN: derived write strengths
    const float *w_f32;                     // diagonal KDN: gains [B, T, H, dk]
    float *dw_out;                          // diagonal KDN: dL/dw [B, T, H, dk]
    const float *invs;                      // diagonal KDN: 1/s [B, T, H] (0 if s = 0)
    float *wdw;                             // diagonal KDN: sum_i w_i dw_i [B, T, H]
    float *pp;                              // diagonal KDN: variance before each token [B,T,H,dk]
    const float *S0;                        // may be null (zero)
    const void *dO;                         // [B, T, H, dv] call dtype
    const float *dS_out;                    // [B, H, dk, dv], may be null (zero)
    float *dq, *dk_, *dv_;                  // [B, T, H, dk / dv]
    float *dla;                             // d log alpha: [B,T,H] (GDN), [B,T,H,dk] (KDA)
    float *dbeta;                           // [B, T, H]
    float *dS0;                             // [B, H, dk, dv], may be null
    const float *dp_out;                    // isotropic KDN: dL/dp_final [B, H], may be null
    float *dxi, *dr, *dp0;                  // isotropic KDN gradients
    void *ws;                               // forward records (kdn_workspace.h)
    int rec_perm;                           // bf16 records in the permuted column order
    void *states;                           // S at every chunk start (call dtype)
    void *dstates;                          // dS leaving every chunk (call dtype)
    // isotropic KDN: the forward variance pass's per-token sums (mean a^2,
    // mean xi, |k|^2, r) and chunk-start variances; the chain's chunk maps
    // and the variance gradient at every chunk end
    const float *ws_stat, *ws_p0;
    float *chain_map, *chain_dp;
    int cus;
};

hipError_t launch_decode(const DecodeParams &P, hipStream_t stream);
hipError_t launch_decode_multi(const DecodeParams &P, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams &P, hipStream_t stream);

// Per-variant prefill launchers (one compilation unit each).
hipError_t launch_prefill_v0(const PrefillParams &P, hipStream_t stream, int nv);
hipError_t launch_prefill_v1(const PrefillParams &P, hipStream_t stream, int nv);
hipError_t launch_prefill_v2(const PrefillParams &P, hipStream_t stream, int nv);
hipError_t launch_prefill_v3(const PrefillParams &P, hipStream_t stream, int nv);
hipError_t launch_prefill_v4(const PrefillParams &P, hipStream_t stream, int nv);

// d_v block width one prefill workgroup owns for this problem.
int prefill_value_block(const PrefillParams &P);

// Two-pass prefill: chunk-parallel prep kernels (one unit per variant), the
// KDN variance scans, and the sequential state pass.
hipError_t launch_prefill_prep_v0(const PrefillParams &P, hipStream_t stream);
hipError_t launch_prefill_prep_v1(const PrefillParams &P, hipStream_t stream);
hipError_t launch_prefill_prep_v2(const PrefillParams &P, hipStream_t stream);
hipError_t launch_prefill_prep_v3(const PrefillParams &P, hipStream_t stream);
hipError_t launch_prefill_prep_v4(const PrefillParams &P, hipStream_t stream);
hipError_t launch_variance_scan(const PrefillParams &P, hipStream_t stream);
hipError_t launch_prefill_state(const PrefillParams &P, hipStream_t stream);
// bf16 state pass on permuted records, one wave per 16-column block
hipError_t launch_prefill_chain(const PrefillParams &P, hipStream_t stream);
// bf16 prefill of short sequences (T <= PREFILL_SHORT_T), one workgroup per
// (batch, head), chunks of 16 tokens
constexpr int PREFILL_SHORT_T = 16;
hipError_t launch_prefill_short(const PrefillParams &P, hipStream_t stream);

// Every argument check of kdn_chunk_prefill except the workspace's own;
// `workspace` tells whether the call has one.  The chunk length in use goes
// to *C_out.  Host only, no HIP call (kdn_abi.cpp).
kdn_status prefill_check(int variant, int dtype, int B, int T, int H, int d_k, int d_v,
                         int chunk, const void *q, const void *k, const void *v,
                         const void *alpha, const void *beta, const void *proc_noise,
                         const void *obs_noise, const float *S0, const float *p0,
                         const void *o, const float *S_out, const float *p_out,
                         bool workspace, int *C_out);

// Bytes of workspace the two-pass schedule needs (0 when there is no chunk).
long long prefill_workspace_bytes(int variant, int bf16, long long B, long long T,
                                  long long H, int dk, int C);

// Gradient kernels (after the forward prep and the state pass with states
// saved): the reverse state pass, then the chunk-parallel local gradients.
hipError_t launch_backward(const BackwardParams &P, hipStream_t stream);

}  // namespace kdn
