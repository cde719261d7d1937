// Device helpers shared by the kernels: storage types, 16-byte row vectors,
// bf16 <-> float32 conversion.  gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace astr {

// bf16 storage as raw 16-bit patterns; arithmetic is always float32.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two floats to packed bf16 with the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32, round to nearest even): lo in bits 0..15.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// A 16-byte slice of a head row: 8 bf16 or 4 float32 elements.
template <typename T> struct Vec;

template <> struct Vec<bf16_t> {
    static constexpr int N = 8;
    uint4 raw;
    __device__ __forceinline__ void load(const bf16_t *p) { raw = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void store(bf16_t *p) const { *reinterpret_cast<uint4 *>(p) = raw; }
    __device__ __forceinline__ void zero() { raw = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void to_float(float (&f)[8]) const {
        f[0] = bf16_lo(raw.x); f[1] = bf16_hi(raw.x);
        f[2] = bf16_lo(raw.y); f[3] = bf16_hi(raw.y);
        f[4] = bf16_lo(raw.z); f[5] = bf16_hi(raw.z);
        f[6] = bf16_lo(raw.w); f[7] = bf16_hi(raw.w);
    }
    __device__ __forceinline__ void from_float(const float (&f)[8]) {
        raw.x = pack_bf16x2(f[0], f[1]);
        raw.y = pack_bf16x2(f[2], f[3]);
        raw.z = pack_bf16x2(f[4], f[5]);
        raw.w = pack_bf16x2(f[6], f[7]);
    }
};

template <> struct Vec<float> {
    static constexpr int N = 4;
    float4 raw;
    __device__ __forceinline__ void load(const float *p) { raw = *reinterpret_cast<const float4 *>(p); }
    __device__ __forceinline__ void store(float *p) const { *reinterpret_cast<float4 *>(p) = raw; }
    __device__ __forceinline__ void zero() { raw = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void to_float(float (&f)[4]) const {
        f[0] = raw.x; f[1] = raw.y; f[2] = raw.z; f[3] = raw.w;
    }
    __device__ __forceinline__ void from_float(const float (&f)[4]) {
        raw = make_float4(f[0], f[1], f[2], f[3]);
    }
};

template <typename T> __device__ __forceinline__ void store_scalar(T *p, float x);
template <> __device__ __forceinline__ void store_scalar<float>(float *p, float x) { *p = x; }
template <> __device__ __forceinline__ void store_scalar<bf16_t>(bf16_t *p, float x) {
    p->bits = static_cast<uint16_t>(f32_to_bf16_bits(x));
}

// 16-byte global load with the non-temporal hint (data read once: KV rows).
__device__ __forceinline__ uint4 load_nt16(const void *p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// exp2(x - m) that is exactly 0 for x = -inf (also when m = -inf).
__device__ __forceinline__ float exp2_sub(float x, float m) {
    return x == -INFINITY ? 0.f : exp2f(x - m);
}

// Rotate one 16-byte slice (E/2 adjacent pairs) by the table entries cs[0..E/2):
// (a, b) -> (a cos - b sin, a sin + b cos), evaluated in float64 (products of
// float32-or-narrower values are exact there), then rounded to float32 and
// stored as T.  The rotary write and the fused decode share it, so both store
// identical bits.
template <typename T>
__device__ __forceinline__ void rotate_slice(Vec<T> &x, const float2 *cs) {
    constexpr int E = Vec<T>::N;
    float f[E];
    x.to_float(f);
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
        const float2 c = cs[j];
        const double a = f[2 * j], b = f[2 * j + 1];
        f[2 * j] = static_cast<float>(a * c.x - b * static_cast<double>(c.y));
        f[2 * j + 1] = static_cast<float>(a * c.y + b * static_cast<double>(c.x));
    }
    x.from_float(f);
}

// KV length of batch entry b, clamped to [0, cap]; 0 when its request row is
// outside the table.  Keeps every req_to_token read inside the table even
// when the device metadata is inconsistent.
__device__ __forceinline__ int request_len(const int32_t *kv_indptr, int b, int req, int num_reqs,
                                           int cap) {
    if (req < 0 || req >= num_reqs) return 0;
    const int L = kv_indptr[b + 1] - kv_indptr[b];
    return L < 0 ? 0 : (L > cap ? cap : L);
}

}  // namespace astr
