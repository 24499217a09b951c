// kdn_device.h -- device-side helpers shared by the gfx950 kernels of this
// library: element conversions, 16-byte vector loads/stores, wave sums and
// the MFMA 16x16 tile step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Variant { DELTANET = 0, GATED_DELTANET = 1, KDA = 2, DIAG_KDN = 3 };

constexpr int WAVE = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even (clang's __bf16 conversion semantics).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) {
    return static_cast<bf16>(x);
}

// Elements of T in one 16-byte vector.
template <typename T> struct Vec16 {
    static constexpr int N = 16 / sizeof(T);
};

// Load N = 16/sizeof(T) consecutive elements (16-byte aligned) as floats.
template <typename T>
__device__ __forceinline__ void load16(const T *p, float (&out)[Vec16<T>::N]);
template <>
__device__ __forceinline__ void load16<float>(const float *p, float (&out)[4]) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
template <>
__device__ __forceinline__ void load16<bf16>(const bf16 *p, float (&out)[8]) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Sum over the 64 lanes of a wave; every lane gets the total.  Fixed
// butterfly order, so results are deterministic.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x += __shfl_xor(x, off, WAVE);
    return x;
}

// ---------------------------------------------------------------------------
// MFMA 16x16 tile step, D(16x16, fp32) += A(16 x KSTEP) * B(KSTEP x 16).
// Operands come from LDS in "k-contiguous" layouts: A as [row][k], B as
// [col][k].  Lane l reads row/col (l & 15) and k offset (l >> 4) * KPL.
// The 16x16 fp32 result sits in 4 registers per lane:
//   acc[r] = D[(l >> 4) * 4 + r][l & 15].
// ---------------------------------------------------------------------------
template <typename E> struct Mma;

template <> struct Mma<bf16> {        // v_mfma_f32_16x16x32_bf16
    static constexpr int KSTEP = 32;
    static constexpr int KPL = 8;     // k elements per lane
    __device__ __forceinline__ static void step(f32x4 &acc, const bf16 *a,
                                                const bf16 *b) {
        const bf16x8 av = *reinterpret_cast<const bf16x8 *>(a);
        const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(b);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
};

template <> struct Mma<float> {       // v_mfma_f32_16x16x4_f32
    static constexpr int KSTEP = 4;
    static constexpr int KPL = 1;
    __device__ __forceinline__ static void step(f32x4 &acc, const float *a,
                                                const float *b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(*a, *b, acc, 0, 0, 0);
    }
};

// acc += A[m0:m0+16, 0:K] * B[0:K, n0:n0+16], A given as [row][k] with
// pitch lda, B as [col][k] with pitch ldb (both in elements).  K must be a
// multiple of Mma<E>::KSTEP.
template <typename E>
__device__ __forceinline__ void mma_tile(f32x4 &acc, const E *A, int lda,
                                         const E *B, int ldb, int K, int lane) {
    const int r = lane & 15;
    const int ko = (lane >> 4) * Mma<E>::KPL;
    const E *pa = A + r * lda + ko;
    const E *pb = B + r * ldb + ko;
    for (int k = 0; k < K; k += Mma<E>::KSTEP)
        Mma<E>::step(acc, pa + k, pb + k);
}

}  // namespace kdn
