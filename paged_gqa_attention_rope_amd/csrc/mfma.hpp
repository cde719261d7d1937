// gfx950 matrix-core and LDS-transpose helpers (bf16 in, float32 accumulate).
//
// v_mfma_f32_16x16x32_bf16, D[i][j] += sum_k A[i][k] B[k][j], lane l of the wave:
//   A: holds A[l % 16][8*(l/16) + e], e = 0..7
//   B: holds B[8*(l/16) + e][l % 16], e = 0..7
//   D: holds D[4*(l/16) + r][l % 16], r = 0..3
// The reduction index k only pairs A with B, so any fixed relabelling of the
// 32 k-slots applied to both operands leaves the product unchanged; the
// kernels use that to make accumulator registers of one product usable as an
// operand of the next.
//
// ds_read_b64_tr_b16: within each group of 16 lanes, with lane j supplying the
// address of 4 consecutive 16-bit elements in[j][0..3], lane i receives
// out[i][e] = in[4e + i/4][i % 4].  If lane j points at row (r0 + j/4),
// column (c0 + 4*(j % 4)) of a row-major bf16 tile M, lane i receives
// M[r0 + e][c0 + i], e = 0..3: four rows of one column -- the transposed
// operand slice an MFMA needs, read straight from a row-major tile.
// (Both layouts were checked on the device with an in-bounds probe.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace astr {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;

union Frag8 {                    // 8 bf16 = one MFMA A or B operand slice
    bf16x8_t v;
    uint4 u;
    uint2 h[2];
    uint32_t w[4];
};

__device__ __forceinline__ f32x4_t mfma16(const Frag8 &a, const Frag8 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

// 8-byte transposing LDS read; `p` must be an 8-byte aligned LDS address.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *p) {
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    const lds_bf16x4 *a = (const lds_bf16x4 *)((const __attribute__((address_space(3))) char *)p);
    union {
        bf16x4_t v;
        uint2 u;
    } r;
    r.v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<lds_bf16x4 *>(a));
    return r.u;
}

// Max over the 4 lanes j, j+16, j+32, j+48 (the same MFMA column in the four
// lane groups).  v_permlane16_swap / v_permlane32_swap applied to (x, x) leave
// each lane with its own value and that of its partner 16 (32) lanes away,
// in one of the two results (checked on the device with an in-bounds probe).
__device__ __forceinline__ float max_over_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Order this wave's LDS writes before its later LDS reads of other lanes'
// data (LDS operations of one wave complete in issue order; this keeps the
// compiler from moving them and waits for the writes).
__device__ __forceinline__ void wave_lds_fence() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// LDS position of 16-byte chunk c of row r of a tile of K or V head rows
// (unpadded, 2*D bytes each): c ^ swz(r).  The XOR swizzle keeps both the
// 128-bit K-operand reads (16 rows, one chunk each) and the transposing V
// reads (4 rows x 32 bytes per 16 lanes) free of LDS bank conflicts (measured
// with the bank-conflict counter), and whole-row writes stay contiguous.
template <int D>
__device__ __forceinline__ constexpr int swz(int r) {
    if constexpr (D == 128) {
        r &= 15;
        return ((r >> 1) ^ (r << 2)) & 15;
    } else {
        return r & 7;
    }
}

}  // namespace astr
