// eda_common.h -- device helpers shared by the EDA kernels (gfx950 only).
//
// Storage types: `bf16` is the raw 16-bit pattern of a bfloat16 (round to
// nearest even on conversion); fp32 is plain float.  Matrix-core products use
// the "NT" convention throughout:
//
//     C[m][n] += sum_k X[m][k] * Y[n][k]
//
// with both X and Y stored row-major with k contiguous.  One 16x16 output
// tile is accumulated by one wavefront (64 lanes).  For lane l the operand
// fragments are X[m0 + l%16][k0 + KPL*(l/16) + 0..KPL-1] and the same for Y
// (KPL = 8 for the bf16 16x16x32 instruction, 1 for fp32 16x16x4); since the
// same k-to-lane map is used for both operands, the sum over k is exact
// whatever order the hardware reduces k in.  The 16x16 fp32 accumulator of
// lane l holds C[4*(l/16) + i][l%16], i = 0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eda {

typedef uint16_t bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Two fp32 -> two bf16 packed in 32 bits (round to nearest even; gfx950 has a
// single instruction for it), low half = a.
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const bf16x2 r = __builtin_convertvector((f32x2{a, b}), bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float lo_bf16(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float(((uint32_t)x) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) {
    return (bf16)(__builtin_bit_cast(uint16_t, (__bf16)x));  // round to nearest even
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }



// ---------------------------------------------------------------------------
// Matrix-core traits.  KB = k consumed per instruction, KPL = k per lane.
// ---------------------------------------------------------------------------
template <typename T> struct MM;

template <> struct MM<bf16> {
    static constexpr int KB = 32, KPL = 8;
    typedef bf16x8 frag;
    static __device__ __forceinline__ frag load(const bf16 *p) {
        return *reinterpret_cast<const bf16x8 *>(p);
    }
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // k = 16 remainder: 16x16x16 instruction, 4 k per lane.
    static __device__ __forceinline__ f32x4 mma16(const bf16 *x, const bf16 *y, f32x4 c) {
        s16x4 a = *reinterpret_cast<const s16x4 *>(x);
        s16x4 b = *reinterpret_cast<const s16x4 *>(y);
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};

template <> struct MM<float> {
    static constexpr int KB = 4, KPL = 1;
    typedef float frag;
    static __device__ __forceinline__ frag load(const float *p) { return *p; }
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// acc += X[0:16][0:K] * Y[0:16][0:K]^T for the wave's 16x16 tile.
// X, Y point at the tile's first row; ldx, ldy are row strides (elements).
template <typename T, int K>
__device__ __forceinline__ f32x4 tile_nt(const T *X, int ldx, const T *Y, int ldy, f32x4 acc,
                                         int lane) {
    static_assert(K % 16 == 0, "tile depth must be a multiple of 16");
    const int r = lane & 15, g = lane >> 4;
    if constexpr (sizeof(T) == 2) {
        constexpr int KF = K / 32 * 32;
        const T *xp = X + r * ldx + 8 * g;
        const T *yp = Y + r * ldy + 8 * g;
#pragma unroll
        for (int k0 = 0; k0 < KF; k0 += 32)
            acc = MM<T>::mma(MM<T>::load(xp + k0), MM<T>::load(yp + k0), acc);
        if constexpr (K % 32 == 16)
            acc = MM<T>::mma16(X + r * ldx + KF + 4 * g, Y + r * ldy + KF + 4 * g, acc);
    } else {
        const T *xp = X + r * ldx + g;
        const T *yp = Y + r * ldy + g;
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += 4)
            acc = MM<T>::mma(xp[k0], yp[k0], acc);
    }
    return acc;
}

// Same, with a run-time depth (multiple of 16 for bf16, of 4 for fp32).
template <typename T>
__device__ __forceinline__ f32x4 tile_nt_dyn(const T *X, int ldx, const T *Y, int ldy, int K,
                                             f32x4 acc, int lane) {
    const int r = lane & 15, g = lane >> 4;
    if constexpr (sizeof(T) == 2) {
        int k0 = 0;
        const T *xp = X + r * ldx + 8 * g;
        const T *yp = Y + r * ldy + 8 * g;
        for (; k0 + 32 <= K; k0 += 32)
            acc = MM<T>::mma(MM<T>::load(xp + k0), MM<T>::load(yp + k0), acc);
        if (k0 < K)
            acc = MM<T>::mma16(X + r * ldx + k0 + 4 * g, Y + r * ldy + k0 + 4 * g, acc);
    } else {
        const T *xp = X + r * ldx + g;
        const T *yp = Y + r * ldy + g;
        for (int k0 = 0; k0 < K; k0 += 4) acc = MM<T>::mma(xp[k0], yp[k0], acc);
    }
    return acc;
}

// acc += A B^T for the wave's 16x16 tile where A is stored TRANSPOSED:
// A[m][k] = M[k][m] with M row-major (k rows, m contiguous).  M points at
// M[k0][m0], Y at Y[n0][k0] (k contiguous).  The gfx950 transposing LDS read
// gives, within each group of 16 lanes where lane i addresses row i/4 and
// columns 4(i%4)..4(i%4)+3 of a 4x16 block, lane n the 4 values of column n
// -- i.e. the A operand of the matrix instruction for 4 consecutive k.
// M must be in LDS.
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
template <int K>
__device__ __forceinline__ f32x4 tile_tn_bf16(const uint16_t *M, int ldm, const uint16_t *Y, int ldy,
                                              f32x4 acc, int lane) {
    static_assert(K % 32 == 0, "tile depth must be a multiple of 32");
    const int g = lane >> 4, i = lane & 15, n = lane & 15;
    const uint16_t *mp = M + (8 * g + (i >> 2)) * ldm + 4 * (i & 3);
    const uint16_t *yp = Y + n * ldy + 8 * g;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(mp + k0 * ldm));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(mp + (k0 + 4) * ldm));
        typedef __attribute__((ext_vector_type(8))) short s16x8;
        const s16x8 a8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a8),
                                                      *reinterpret_cast<const bf16x8 *>(yp + k0), acc, 0, 0, 0);
    }
    return acc;
}

// Store 4 consecutive values (one accumulator's column run) as T.
template <typename T> __device__ __forceinline__ void store4(T *p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<bf16>(bf16 *p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16(a, b), pack_bf16(c, d));
}
template <> __device__ __forceinline__ void store4<float>(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{a, b, c, d};
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

}  // namespace eda
