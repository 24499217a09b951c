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

enum Variant { DELTANET = 0, GATED_DELTANET = 1, KDA = 2, DIAG_KDN = 3, ISO_KDN = 4 };

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

// Sum over each row of 16 lanes by DPP row shifts (no LDS traffic); lane 15
// of the row holds the total, the other lanes partial sums.
__device__ __forceinline__ float row16_sum_last(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
    return x;
}

// Sum over each group of 8 lanes by DPP row shifts; lane 7 of the group
// holds the total.
__device__ __forceinline__ float row8_sum_last(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
    return x;
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

// K = 16 step for small products (the triangular-inverse blocks).
template <typename E> struct Mma16;

template <> struct Mma16<bf16> {      // v_mfma_f32_16x16x16_bf16
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    // A: [row][k] pitch lda, rows (lane & 15), k = (lane >> 4) * 4 .. + 3
    __device__ __forceinline__ static void tile(f32x4 &acc, const bf16 *A, int lda,
                                                const bf16 *B, int ldb, int lane) {
        const int r = lane & 15, ko = (lane >> 4) * 4;
        const s16x4 av = *reinterpret_cast<const s16x4 *>(A + r * lda + ko);
        const s16x4 bv = *reinterpret_cast<const s16x4 *>(B + r * ldb + ko);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, acc, 0, 0, 0);
    }
};

template <> struct Mma16<float> {     // 4 x v_mfma_f32_16x16x4_f32
    __device__ __forceinline__ static void tile(f32x4 &acc, const float *A, int lda,
                                                const float *B, int ldb, int lane) {
        const int r = lane & 15, ko = lane >> 4;
        float a[4], b[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            a[s] = A[r * lda + ko + 4 * s];
            b[s] = B[r * ldb + ko + 4 * s];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    }
};

// As mma_tile with a compile-time K: every operand load is issued before the
// first MFMA so the LDS latency is paid once per tile.
template <typename E, int K>
__device__ __forceinline__ void mma_tile_k(f32x4 &acc, const E *A, int lda,
                                           const E *B, int ldb, int lane) {
    constexpr int NS = K / Mma<E>::KSTEP;
    static_assert(NS * Mma<E>::KSTEP == K, "K multiple of the MFMA step");
    const int r = lane & 15;
    const int ko = (lane >> 4) * Mma<E>::KPL;
    const E *pa = A + r * lda + ko;
    const E *pb = B + r * ldb + ko;
    if constexpr (sizeof(E) == 2) {
        bf16x8 av[NS], bv[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            av[s] = *reinterpret_cast<const bf16x8 *>(pa + s * Mma<E>::KSTEP);
            bv[s] = *reinterpret_cast<const bf16x8 *>(pb + s * Mma<E>::KSTEP);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[s], bv[s], acc, 0, 0, 0);
    } else {
        float av[NS], bv[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            av[s] = pa[s * Mma<E>::KSTEP];
            bv[s] = pb[s * Mma<E>::KSTEP];
        }
#pragma unroll
        for (int s = 0; s < NS; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc, 0, 0, 0);
    }
}

// Eight consecutive elements of E in LDS (16-byte aligned) as floats.
__device__ __forceinline__ void lds_ld8(const bf16 *p, float (&f)[8]) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void lds_ld8(const float *p, float (&f)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void lds_st8(bf16 *p, const float (&f)[8]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = static_cast<bf16>(f[i]);
    *reinterpret_cast<bf16x8 *>(p) = v;
}
__device__ __forceinline__ void lds_st8(float *p, const float (&f)[8]) {
    *reinterpret_cast<float4 *>(p) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}
// N (1, 2 or 4) consecutive elements of E in LDS, aligned to N elements.
template <int N>
__device__ __forceinline__ void lds_stn(bf16 *p, const float *f) {
    if constexpr (N == 2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 v;
        v[0] = static_cast<bf16>(f[0]); v[1] = static_cast<bf16>(f[1]);
        *reinterpret_cast<bf16x2 *>(p) = v;
    } else if constexpr (N == 4) {
        bf16x4 v;
        v[0] = static_cast<bf16>(f[0]); v[1] = static_cast<bf16>(f[1]);
        v[2] = static_cast<bf16>(f[2]); v[3] = static_cast<bf16>(f[3]);
        *reinterpret_cast<bf16x4 *>(p) = v;
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            p[i] = static_cast<bf16>(f[i]);
    }
}
template <int N>
__device__ __forceinline__ void lds_stn(float *p, const float *f) {
    if constexpr (N == 2) {
        *reinterpret_cast<float2 *>(p) = make_float2(f[0], f[1]);
    } else if constexpr (N == 4) {
        *reinterpret_cast<float4 *>(p) = make_float4(f[0], f[1], f[2], f[3]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            p[i] = f[i];
    }
}

// Fast reciprocal (v_rcp_f32, about 1 ulp).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Kalman variance step as a linear fractional map of the variance p, held as
// a 2 x 2 matrix acting on (p, 1) projectively (page "给记忆装一个信任度探测器：
// Kalman Delta Networks ...", sections "对角近似：把矩阵压扁成一个向量" and
// "各向同性近似：把整个头压缩成一个数": the recursion is a Mobius map and runs of
// tokens compose by matrix products).  Entries are >= 0 for admissible
// inputs, so products have no cancellation and may be rescaled freely.
struct Map2 {
    float a, b, c, d;     // [[a, b], [c, d]]
    // x <- y o x (y applied after x)
    __device__ __forceinline__ void after(float ya, float yb, float yc, float yd) {
        const float na = ya * a + yb * c, nb = ya * b + yb * d;
        const float nc = yc * a + yd * c, nd = yc * b + yd * d;
        a = na; b = nb; c = nc; d = nd;
    }
    // x <- x o y (y applied first)
    __device__ __forceinline__ void before(float ya, float yb, float yc, float yd) {
        const float na = a * ya + b * yc, nb = a * yb + b * yd;
        const float nc = c * ya + d * yc, nd = c * yb + d * yd;
        a = na; b = nb; c = nc; d = nd;
    }
    // divide by the largest entry (the map is unchanged by a common factor)
    __device__ __forceinline__ void rescale() {
        const float sc = fast_rcp(fmaxf(fmaxf(a, b), fmaxf(c, d)));
        a *= sc; b *= sc; c *= sc; d *= sc;
    }
    __device__ __forceinline__ float apply(float p) const {
        return fmaf(a, p, b) / fmaf(c, p, d);
    }
};

// One token: predict p- = a2 p + xi, then p = p- r / (r + m p-), where m is
// the precision gain numerator (mu k_i^2 per channel, or (mu / d_k) |k|^2 for
// one variance per head).  Divided through by r:
//   [[a2, xi], [c a2, c xi + 1]],  c = m / r   (r > 0);
// r = 0: the identity update if m = 0 ([[a2, xi], [0, 1]]), else every p-
// maps to 0 ([[0, 0], [0, 1]]).
__device__ __forceinline__ Map2 variance_step_map(float a2, float xi, float m, float r) {
    Map2 y{a2, xi, 0.f, 1.f};
    if (r > 0.f) {
        const float cc = m / r;
        y.c = cc * a2;
        y.d = fmaf(cc, xi, 1.f);
    } else if (m != 0.f) {
        y.a = 0.f;
        y.b = 0.f;
    }
    return y;
}

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
