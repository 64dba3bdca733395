// Device helpers shared by the conv1d and selective-scan kernels (gfx950).
//
// Element storage: float32 or bf16 (raw 16-bit patterns).  bf16 -> f32 is a
// 16-bit shift; f32 -> bf16 rounds to nearest even (the compiler lowers the
// __bf16 conversion to the gfx950 hardware convert).
//
// Transcendentals use the hardware base-2 instructions (v_exp_f32, v_log_f32,
// v_rcp_f32), each about 1 ulp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mamba {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

// Load / store one element of storage type T as float.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
    __device__ __forceinline__ static float load(const void* p, int64_t i) {
        return static_cast<const float*>(p)[i];
    }
    __device__ __forceinline__ static void store(void* p, int64_t i, float v) {
        static_cast<float*>(p)[i] = v;
    }
};
template <> struct Elem<bf16_t> {
    static constexpr int kBytes = 2;
    __device__ __forceinline__ static float load(const void* p, int64_t i) {
        return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    }
    __device__ __forceinline__ static void store(void* p, int64_t i, float v) {
        static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    }
};

// VEC consecutive elements of one token row as floats: 16-byte vectors (8 bf16 or
// 4 f32 channels), 8-byte vectors (4 bf16 channels) or single elements (ragged
// D, unaligned buffers).
template <typename T, int VEC> struct VecIO;

// bf16, 8 channels = 16 bytes
template <> struct VecIO<bf16_t, 8> {
    __device__ __forceinline__ static void load(const void* base, int64_t off, float (&v)[8]) {
        const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static void store(void* base, int64_t off, const float (&v)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
                   (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = make_uint4(w[0], w[1], w[2], w[3]);
    }
};

// bf16, 4 channels = 8 bytes
template <> struct VecIO<bf16_t, 4> {
    __device__ __forceinline__ static void load(const void* base, int64_t off, float (&v)[4]) {
        const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
        v[0] = __uint_as_float(raw.x << 16);
        v[1] = __uint_as_float(raw.x & 0xffff0000u);
        v[2] = __uint_as_float(raw.y << 16);
        v[3] = __uint_as_float(raw.y & 0xffff0000u);
    }
    __device__ __forceinline__ static void store(void* base, int64_t off, const float (&v)[4]) {
        const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
        const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + off) = make_uint2(lo, hi);
    }
};

// f32, 4 channels = 16 bytes
template <> struct VecIO<float, 4> {
    __device__ __forceinline__ static void load(const void* base, int64_t off, float (&v)[4]) {
        const float4 raw = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
        v[0] = raw.x; v[1] = raw.y; v[2] = raw.z; v[3] = raw.w;
    }
    __device__ __forceinline__ static void store(void* base, int64_t off, const float (&v)[4]) {
        *reinterpret_cast<float4*>(static_cast<float*>(base) + off) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

// Any type, 1 channel (ragged D or unaligned buffers).
template <typename T> struct VecIO<T, 1> {
    __device__ __forceinline__ static void load(const void* base, int64_t off, float (&v)[1]) {
        v[0] = Elem<T>::load(base, off);
    }
    __device__ __forceinline__ static void store(void* base, int64_t off, const float (&v)[1]) {
        Elem<T>::store(base, off, v[0]);
    }
};

// SiLU(v) = v * sigmoid(v) = v / (1 + 2^(-v log2 e)).  For very negative v the
// exponential overflows to +inf and the reciprocal gives 0, so the result is -0.
__device__ __forceinline__ float silu_f(float v) {
    return v * rcp_fast(1.0f + exp2_fast(-v * kLog2e));
}

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|).
// With y = e^-|v| in (0, 1]: for |v| > 4 (y < 0.0184) log1p(y) uses its series
// to the y^5 term (truncation below 7e-12 relative); otherwise log2(1 + y) ln 2,
// where 1 + y >= 1.018 keeps the rounding of 1 + y harmless.  This keeps small
// step sizes (dt near 1e-3, the low end of the usual dt range) accurate to a
// few ulp, where log(1 + e^v) evaluated directly would lose ~3 digits.
__device__ __forceinline__ float softplus_f(float v) {
    const float av = __builtin_fabsf(v);
    const float y = exp2_fast(-av * kLog2e);
    const float series =
        y * __builtin_fmaf(-y, __builtin_fmaf(-y, __builtin_fmaf(-y, __builtin_fmaf(-y, 0.2f, 0.25f),
                                                                  0.33333334f), 0.5f), 1.0f);
    const float direct = log2_fast(1.0f + y) * kLn2;
    return __builtin_fmaxf(v, 0.0f) + (av > 4.0f ? series : direct);
}

}  // namespace mamba
