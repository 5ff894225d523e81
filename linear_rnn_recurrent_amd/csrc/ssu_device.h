// Device-side helpers shared by the SSU kernels: dtype conversions, 16-byte
// state-vector loads/stores, small wave64 lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssu {

enum : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A buffer pointer read from a device-side table is generic to the compiler,
// so accesses through it become flat instructions (which also count against
// the LDS/scalar wait counter). Converting its address to a global-memory
// pointer lets them compile to global instructions: valid for every buffer the
// library accepts (device or host-mapped memory, never LDS or scratch), whose
// global and generic addresses are the same.
template <typename T>
__device__ __forceinline__ T *table_ptr(const void *p)
{
    return (T *)(__attribute__((address_space(1))) T *)reinterpret_cast<uintptr_t>(p);
}

// Storage tag for a bf16 state element (no arithmetic is done on it).
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// fptrunc in the default round-to-nearest-even mode.
__device__ __forceinline__ uint32_t f32_to_f16(float f)
{
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float lo16(uint32_t w, int dt)
{
    return dt == kBF16 ? __uint_as_float(w << 16) : f16_to_f32(w & 0xffffu);
}
__device__ __forceinline__ float hi16(uint32_t w, int dt)
{
    return dt == kBF16 ? __uint_as_float(w & 0xffff0000u) : f16_to_f32(w >> 16);
}

// Scalar element of an x/z/out tensor in io dtype.
__device__ __forceinline__ float ld_io(const void *p, int64_t i, int dt)
{
    if (dt == kF32)
        return static_cast<const float *>(p)[i];
    const uint32_t h = static_cast<const uint16_t *>(p)[i];
    return dt == kBF16 ? bf16_to_f32(h) : f16_to_f32(h);
}

__device__ __forceinline__ void st_io(void *p, int64_t i, float v, int dt)
{
    if (dt == kF32)
        static_cast<float *>(p)[i] = v;
    else
        static_cast<uint16_t *>(p)[i] = (uint16_t)(dt == kBF16 ? f32_to_bf16(v) : f32_to_f16(v));
}

// Typed scalar element access for x/z/out tensors whose dtype is a template
// parameter (float, _Float16 or bf16_t): one load or store, no branch.
template <typename T>
__device__ __forceinline__ float ld_elem(const void *p, int64_t i)
{
    if constexpr (sizeof(T) == 4) {
        return static_cast<const float *>(p)[i];
    } else {
        const uint32_t h = static_cast<const uint16_t *>(p)[i];
        if constexpr (__is_same(T, bf16_t))
            return bf16_to_f32(h);
        else
            return f16_to_f32(h);
    }
}

template <typename T>
__device__ __forceinline__ void st_elem(void *p, int64_t i, float v)
{
    if constexpr (sizeof(T) == 4)
        static_cast<float *>(p)[i] = v;
    else if constexpr (__is_same(T, bf16_t))
        static_cast<uint16_t *>(p)[i] = (uint16_t)f32_to_bf16(v);
    else
        static_cast<uint16_t *>(p)[i] = (uint16_t)f32_to_f16(v);
}

// Four consecutive elements at element offset i (base aligned to four
// elements), rounded as st_elem rounds them, in one store.
template <typename T>
__device__ __forceinline__ void st_raw4(void *p, uint32_t i, const float (&v)[4])
{
    if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<float4 *>(static_cast<float *>(p) + i) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
        uint32_t h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            h[k] = __is_same(T, bf16_t) ? f32_to_bf16(v[k]) : f32_to_f16(v[k]);
        *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p) + i) =
            u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    }
}

// N consecutive B/C elements (N a multiple of 4) of storage type T at element
// offset i (a multiple of N; base 16-byte aligned), loaded as whole vectors
// before any conversion so that the loads are all in flight together.
template <typename T, int N>
__device__ __forceinline__ void ld_typed(const void *p, int64_t i, float (&v)[N])
{
    static_assert(N % 4 == 0, "N must be a multiple of 4");
    if constexpr (sizeof(T) == 4) {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(static_cast<const float *>(p) + i);
        u32x4 w[N / 4];
#pragma unroll
        for (int k = 0; k < N / 4; ++k)
            w[k] = q[k];
#pragma unroll
        for (int k = 0; k < N / 4; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[4 * k + j] = __uint_as_float(w[k][j]);
    } else if constexpr (N % 8 != 0) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(p) + i);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (__is_same(T, bf16_t)) {
                v[2 * j] = __uint_as_float(w[j] << 16);
                v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            } else {
                v[2 * j] = f16_to_f32(w[j] & 0xffffu);
                v[2 * j + 1] = f16_to_f32(w[j] >> 16);
            }
        }
    } else {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p) + i);
        u32x4 w[N / 8];
#pragma unroll
        for (int k = 0; k < N / 8; ++k)
            w[k] = q[k];
#pragma unroll
        for (int k = 0; k < N / 8; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (__is_same(T, bf16_t)) {
                    v[8 * k + 2 * j] = __uint_as_float(w[k][j] << 16);
                    v[8 * k + 2 * j + 1] = __uint_as_float(w[k][j] & 0xffff0000u);
                } else {
                    v[8 * k + 2 * j] = f16_to_f32(w[k][j] & 0xffffu);
                    v[8 * k + 2 * j + 1] = f16_to_f32(w[k][j] >> 16);
                }
            }
    }
}

// Raw (unconverted) loads for prefetching: the value is kept as bits until it
// is converted, so no wait is forced at the load. raw4: 4 consecutive elements
// (element offset a multiple of 4, base 16-byte aligned).
template <typename T>
struct Raw4 {
    typedef u32x2 type;  // four 16-bit elements
};
template <>
struct Raw4<float> {
    typedef u32x4 type;
};

template <typename T>
__device__ __forceinline__ typename Raw4<T>::type ld_raw4(const void *p, int64_t i)
{
    if constexpr (sizeof(T) == 4)
        return *reinterpret_cast<const u32x4 *>(static_cast<const float *>(p) + i);
    else
        return *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(p) + i);
}

template <typename T>
__device__ __forceinline__ void cvt_raw4(const typename Raw4<T>::type w, float (&v)[4])
{
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = __uint_as_float(w[j]);
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (__is_same(T, bf16_t)) {
                v[2 * j] = __uint_as_float(w[j] << 16);
                v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            } else {
                v[2 * j] = f16_to_f32(w[j] & 0xffffu);
                v[2 * j + 1] = f16_to_f32(w[j] >> 16);
            }
        }
    }
}

// One element as raw bits (zero-extended for 16-bit types), and its conversion.
template <typename T>
__device__ __forceinline__ uint32_t ld_raw1(const void *p, int64_t i)
{
    if constexpr (sizeof(T) == 4)
        return static_cast<const uint32_t *>(p)[i];
    else
        return static_cast<const uint16_t *>(p)[i];
}

template <typename T>
__device__ __forceinline__ float cvt_raw1(uint32_t w)
{
    if constexpr (sizeof(T) == 4)
        return __uint_as_float(w);
    else if constexpr (__is_same(T, bf16_t))
        return __uint_as_float(w << 16);
    else
        return f16_to_f32(w);
}

// N consecutive elements (N a multiple of 4) of a B/C-like tensor at element
// offset i, which is a multiple of 4 (of 8 when N is); the base is 16-byte
// aligned. When i is the same on every lane the loads are wave-uniform and the
// compiler keeps them on the scalar unit.
template <int N>
__device__ __forceinline__ void ld_vec(const void *p, int64_t i, int dt, float (&v)[N])
{
    static_assert(N % 4 == 0, "N must be a multiple of 4");
    if (dt == kF32) {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(static_cast<const float *>(p) + i);
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            const u32x4 w = q[k];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[4 * k + j] = __uint_as_float(w[j]);
        }
    } else if constexpr (N % 8 != 0) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(p) + i);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            v[2 * j] = lo16(w[j], dt);
            v[2 * j + 1] = hi16(w[j], dt);
        }
    } else {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p) + i);
#pragma unroll
        for (int k = 0; k < N / 8; ++k) {
            const u32x4 w = q[k];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * k + 2 * j] = lo16(w[j], dt);
                v[8 * k + 2 * j + 1] = hi16(w[j], dt);
            }
        }
    }
}

// N consecutive B/C elements of storage type BT (float, _Float16 or bf16_t)
// at element offset i (a multiple of 8; base 16-byte aligned). Used with a
// wave-uniform offset inside the prefill token loop, where the dtype is a
// template parameter so that only one conversion path is emitted.
template <typename BT, int N>
__device__ __forceinline__ void ld_bc(const void *p, int64_t i, float (&v)[N])
{
    static_assert(N % 8 == 0, "N must be a multiple of 8");
    if constexpr (sizeof(BT) == 4) {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(static_cast<const float *>(p) + i);
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            const u32x4 w = q[k];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[4 * k + j] = __uint_as_float(w[j]);
        }
    } else {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p) + i);
#pragma unroll
        for (int k = 0; k < N / 8; ++k) {
            const u32x4 w = q[k];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (sizeof(BT) == 2 && __is_same(BT, bf16_t)) {
                    v[8 * k + 2 * j] = __uint_as_float(w[j] << 16);
                    v[8 * k + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
                } else {
                    v[8 * k + 2 * j] = f16_to_f32(w[j] & 0xffffu);
                    v[8 * k + 2 * j + 1] = f16_to_f32(w[j] >> 16);
                }
            }
        }
    }
}

__device__ __forceinline__ int clamp_len(int v, int hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

// 16-byte state vectors: 4 fp32 or 8 fp16/bf16 elements.
template <typename ST>
struct SV;

template <>
struct SV<float> {
    static constexpr int VEC = 4;
    __device__ static __forceinline__ void unpack(const u32x4 w, float (&v)[4])
    {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = __uint_as_float(w[j]);
    }
    __device__ static __forceinline__ u32x4 pack(const float (&v)[4])
    {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = __float_as_uint(v[j]);
        return w;
    }
};

template <>
struct SV<_Float16> {
    static constexpr int VEC = 8;
    __device__ static __forceinline__ void unpack(const u32x4 w, float (&v)[8])
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = f16_to_f32(w[j] & 0xffffu);
            v[2 * j + 1] = f16_to_f32(w[j] >> 16);
        }
    }
    __device__ static __forceinline__ u32x4 pack(const float (&v)[8])
    {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = f32_to_f16(v[2 * j]) | (f32_to_f16(v[2 * j + 1]) << 16);
        return w;
    }
};

template <>
struct SV<bf16_t> {
    static constexpr int VEC = 8;
    __device__ static __forceinline__ void unpack(const u32x4 w, float (&v)[8])
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
    __device__ static __forceinline__ u32x4 pack(const float (&v)[8])
    {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = f32_to_bf16(v[2 * j]) | (f32_to_bf16(v[2 * j + 1]) << 16);
        return w;
    }
};

__device__ __forceinline__ float softplus_f32(float v)
{
    // log(1 + e^v), a few ulp, on the hardware exp2 / log2 / rcp. Above 20 the
    // correction e^-v is below the fp32 resolution of v. log1p(e) as
    // log(u) e / (u - 1) with u = 1 + e (the rounding of u cancels: Goldberg's
    // method); below 2^-24 (u == 1) log1p(e) is e itself.
    const float e = __builtin_amdgcn_exp2f(v * 1.4426950408889634f);
    const float u = 1.0f + e;
    const float l = u == 1.0f ? e
                              : __builtin_amdgcn_logf(u) * 0.6931471805599453f * e *
                                    __builtin_amdgcn_rcpf(u - 1.0f);
    return v > 20.0f ? v : l;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64);
// every lane of a group receives the group sum.
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int m = 1; m < W; m <<= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

}  // namespace ssu
