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
#include <type_traits>
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

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for every
// outstanding global load and store of the wave, which would expose the memory
// latency at each barrier of a chunk loop (stores to drain, prefetches to land);
// here the wave waits for its own LDS operations (lgkmcnt) and then meets the
// others.  Global data a wave stores is never read back by another wave of the
// same launch in these kernels.  The "memory" clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Inclusive prefix sum over the lanes of a wave64 (lane i gets x_0 + ... + x_i),
// in DPP moves that stay in the vector ALU (a __shfl_up ladder goes through
// ds_bpermute and waits on LDS at each of its six steps).  Hillis-Steele inside
// each row of 16 lanes (row_shr 1, 2, 4, 8; a lane without a source reads the
// identity 0), then row_bcast:15 adds lane 15 of each row to the next row (rows
// 1 and 3) and row_bcast:31 adds lane 31 to rows 2 and 3.
__device__ __forceinline__ float wave_prefix_sum(float x) {
    auto shifted = [](float v, auto ctrl, auto row_mask) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     decltype(ctrl)::value,
                                                                     decltype(row_mask)::value, 0xf, false));
    };
    using I = int;
    x += shifted(x, std::integral_constant<I, 0x111>{}, std::integral_constant<I, 0xf>{});   // row_shr:1
    x += shifted(x, std::integral_constant<I, 0x112>{}, std::integral_constant<I, 0xf>{});   // row_shr:2
    x += shifted(x, std::integral_constant<I, 0x114>{}, std::integral_constant<I, 0xf>{});   // row_shr:4
    x += shifted(x, std::integral_constant<I, 0x118>{}, std::integral_constant<I, 0xf>{});   // row_shr:8
    x += shifted(x, std::integral_constant<I, 0x142>{}, std::integral_constant<I, 0xa>{});   // row_bcast:15
    x += shifted(x, std::integral_constant<I, 0x143>{}, std::integral_constant<I, 0xc>{});   // row_bcast:31
    return x;
}

// The same inside each row of 16 lanes only (lane i gets the sum over lanes
// 16 (i / 16) .. i).
__device__ __forceinline__ float row16_prefix_sum(float x) {
    auto shifted = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     decltype(ctrl)::value, 0xf, 0xf, false));
    };
    using I = int;
    x += shifted(x, std::integral_constant<I, 0x111>{});
    x += shifted(x, std::integral_constant<I, 0x112>{});
    x += shifted(x, std::integral_constant<I, 0x114>{});
    x += shifted(x, std::integral_constant<I, 0x118>{});
    return x;
}

// Inclusive suffix sum inside each row of 16 lanes (lane i gets the sum over
// lanes i .. 16 (i / 16) + 15): row_shl 1, 2, 4, 8.
__device__ __forceinline__ float row16_suffix_sum(float x) {
    auto shifted = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     decltype(ctrl)::value, 0xf, 0xf, false));
    };
    using I = int;
    x += shifted(x, std::integral_constant<I, 0x101>{});
    x += shifted(x, std::integral_constant<I, 0x102>{});
    x += shifted(x, std::integral_constant<I, 0x104>{});
    x += shifted(x, std::integral_constant<I, 0x108>{});
    return x;
}

// Sum over aligned groups of G consecutive lanes (G = 2, 4 or 8), every lane of a
// group getting the group's sum: DPP quad_perm swaps of neighbours and pairs,
// then row_half_mirror (lane i of an 8-lane half-row reads lane 7 - i, in the
// other quad).
template <int G>
__device__ __forceinline__ float lane_group_sum(float x) {
    static_assert(G == 2 || G == 4 || G == 8, "groups inside a DPP half-row");
    auto moved = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     decltype(ctrl)::value, 0xf, 0xf, false));
    };
    using I = int;
    x += moved(x, std::integral_constant<I, 0xB1>{});               // quad_perm [1, 0, 3, 2]
    if constexpr (G >= 4) x += moved(x, std::integral_constant<I, 0x4E>{});   // quad_perm [2, 3, 0, 1]
    if constexpr (G >= 8) x += moved(x, std::integral_constant<I, 0x141>{});  // row_half_mirror
    return x;
}

// Lane `src`'s value of x in every lane (v_readlane: a scalar register).
__device__ __forceinline__ float lane_value(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src));
}

// Two floats to a packed pair of bf16 (lo in bits 0..15), rounded to nearest
// even: one v_cvt_pk_bf16_f32 on gfx950 (two scalar conversions and a merge
// otherwise).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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
            w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
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
        const uint32_t lo = pack_bf16x2(v[0], v[1]);
        const uint32_t hi = pack_bf16x2(v[2], v[3]);
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
// With y = e^-|v| in (0, 1] and u = 1 + y rounded to float, c = (u - 1) - y is
// exactly the rounding error of 1 + y, and log1p(y) = log(u) - c/u + O(c^2);
// taking -c for -c/u errs by c y / u <= 2^-24 y, i.e. below one ulp of
// log1p(y) ~ y.  So small step sizes (dt near 1e-3, y near 1e-3) keep full
// relative accuracy without a separate series, for 9 VALU slots of arithmetic
// after the exponential.
__device__ __forceinline__ float softplus_f(float v) {
    const float y = exp2_fast(-__builtin_fabsf(v) * kLog2e);
    const float u = 1.0f + y;
    const float c = (u - 1.0f) - y;
    return __builtin_fmaxf(v, 0.0f) + __builtin_fmaf(log2_fast(u), kLn2, -c);
}

}  // namespace mamba
