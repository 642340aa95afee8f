// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round-to-nearest-even float -> bfloat16 (finite inputs).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

// Element traits: how a stored element converts to and from fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float to_f32(float v) { return v; }
    __device__ __forceinline__ static float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
    __device__ __forceinline__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
    __device__ __forceinline__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// 16 bytes of operand per lane feed one 16x16 MFMA block over a 64-byte
// K slab: 32 bf16 (one v_mfma_f32_16x16x32_bf16) or 16 fp32 (four
// v_mfma_f32_16x16x4_f32).  Lane l carries row (l % 16) and the 16-byte
// chunk (l / 16) of the slab for both operands, so both operands see the
// same permutation of K and the dot product is unchanged.
template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
    static constexpr int kSlabElems = 32;
    __device__ __forceinline__ static f32x4 run(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static constexpr int kSlabElems = 16;
    __device__ __forceinline__ static f32x4 run(uint4 a, uint4 b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
        return c;
    }
};

__device__ __forceinline__ uint4 ldg16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void stg16(void* p, uint4 v) {
    *reinterpret_cast<uint4*>(p) = v;
}

// Eight values of type T packed in 16 (bf16) or 32 (fp32) bytes, to fp32.
__device__ __forceinline__ void unpack8(const bf16_t* p, float (&o)[8]) {
    uint4 v = ldg16(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack8(const float* p, float (&o)[8]) {
    uint4 a = ldg16(p), b = ldg16(p + 4);
    o[0] = __uint_as_float(a.x); o[1] = __uint_as_float(a.y);
    o[2] = __uint_as_float(a.z); o[3] = __uint_as_float(a.w);
    o[4] = __uint_as_float(b.x); o[5] = __uint_as_float(b.y);
    o[6] = __uint_as_float(b.z); o[7] = __uint_as_float(b.w);
}
__device__ __forceinline__ void pack8(bf16_t* p, const float (&v)[8]) {
    uint4 r;
    r.x = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    r.y = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
    r.z = f32_to_bf16(v[4]) | (static_cast<uint32_t>(f32_to_bf16(v[5])) << 16);
    r.w = f32_to_bf16(v[6]) | (static_cast<uint32_t>(f32_to_bf16(v[7])) << 16);
    stg16(p, r);
}
__device__ __forceinline__ void pack8(float* p, const float (&v)[8]) {
    stg16(p, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]),
                        __float_as_uint(v[2]), __float_as_uint(v[3])));
    stg16(p + 4, make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]),
                            __float_as_uint(v[6]), __float_as_uint(v[7])));
}

}  // namespace moe
