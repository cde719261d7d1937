// Rotary position embedding fused with the KV-cache write, and its gradient.
//
// AstrAI docs/developer/internals.md, "Rotary Position Embedding (RoPE)" and
// "KV Cache Mathematics": q and k are rotated by their token's position and
// the rotated k is what enters the cache (rotation before the write, so cached
// keys keep the rotation of their own position).  docs/guides/inference.md,
// "Rotary Embedding Backend": one fused kernel looks up cos/sin in the
// [max_len, dim/2, 2] float32 table and rotates; adjacent elements
// (x[2i], x[2i+1]) form the complex number that is multiplied.
//
// The whole path is bandwidth-bound (~10 flop per 16 bytes), so the kernel is
// a flat grid of 16-byte vectors: each thread owns one 16-byte slice of one
// head row (8 bf16 or 4 float32 = 4 or 2 rotation pairs), reads it and the
// matching 32 or 16 bytes of the table, and writes 16 bytes.  Consecutive
// threads cover consecutive slices of a row, so every load and store is a
// fully coalesced 16-byte access.
#include "device.hpp"
#include "kernels.hpp"

namespace astr {
namespace {

__global__ __launch_bounds__(256) void rope_table_kernel(float2 *__restrict__ tab, int max_pos,
                                                         int half, double theta) {
    int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= static_cast<int64_t>(max_pos) * half) return;
    int i = static_cast<int>(gid % half);
    int64_t pos = gid / half;
    // w_i = theta^(-2i/d) and the angle in float64: at positions near 32k a
    // float32 angle would be off by ~2e-3 rad.
    double w = pow(theta, (-2.0 * static_cast<double>(i)) / static_cast<double>(2 * half));
    double a = static_cast<double>(pos) * w;
    tab[gid] = make_float2(static_cast<float>(cos(a)), static_cast<float>(sin(a)));
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kv_write_kernel(
    T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const int32_t *__restrict__ positions, const int32_t *__restrict__ loc, int n_tokens,
    int n_heads, int n_kv, const float2 *__restrict__ tab, int max_pos, T *__restrict__ k_layer,
    T *__restrict__ v_layer, int64_t pool_slots) {
    constexpr int E = Vec<T>::N;      // elements per 16-byte slice
    constexpr int VPR = D / E;        // slices per head row
    const int heads_all = n_heads + 2 * n_kv;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= static_cast<int64_t>(n_tokens) * heads_all * VPR) return;
    const int vi = static_cast<int>(gid % VPR);
    const int64_t r = gid / VPR;
    const int hh = static_cast<int>(r % heads_all);
    const int t = static_cast<int>(r / heads_all);
    const int pos = positions[t];
    const int64_t slot = loc[t];
    if (pos < 0 || pos >= max_pos || slot < 0 || slot >= pool_slots) return;

    if (hh >= n_heads + n_kv) {       // v: plain copy into the pool
        const int h = hh - n_heads - n_kv;
        Vec<T> x;
        x.load(v + (static_cast<int64_t>(t) * n_kv + h) * D + vi * E);
        x.store(v_layer + (slot * n_kv + h) * D + vi * E);
        return;
    }
    const T *src;
    T *dst;
    if (hh < n_heads) {               // q: rotated in place
        src = q + (static_cast<int64_t>(t) * n_heads + hh) * D + vi * E;
        dst = q + (static_cast<int64_t>(t) * n_heads + hh) * D + vi * E;
    } else {                          // k: rotated, then written to the pool
        const int h = hh - n_heads;
        src = k + (static_cast<int64_t>(t) * n_kv + h) * D + vi * E;
        dst = k_layer + (slot * n_kv + h) * D + vi * E;
    }
    // float64 arithmetic: a*cos and b*sin of float32-or-narrower operands are
    // exact, so the stored value is the correctly rounded rotation by the
    // table even when a*cos and b*sin nearly cancel
    Vec<T> x;
    x.load(src);
    rotate_slice(x, tab + static_cast<int64_t>(pos) * (D / 2) + vi * (E / 2));
    x.store(dst);
}

// Gradient of the rotation, in place: each pair is multiplied by the complex
// conjugate of the forward table entry (the exact transpose of the forward
// map), evaluated in float64 and rounded once, as forward.
template <typename T, int D>
__global__ __launch_bounds__(256) void rope_backward_kernel(T *__restrict__ grad,
                                                            const int32_t *__restrict__ positions,
                                                            int n_tokens, int n_heads,
                                                            const float2 *__restrict__ tab, int max_pos) {
    constexpr int E = Vec<T>::N;      // elements per 16-byte slice
    constexpr int VPR = D / E;        // slices per head row
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= static_cast<int64_t>(n_tokens) * n_heads * VPR) return;
    const int vi = static_cast<int>(gid % VPR);
    const int t = static_cast<int>(gid / VPR / n_heads);
    const int pos = positions[t];
    if (pos < 0 || pos >= max_pos) return;
    T *p = grad + (gid / VPR) * D + vi * E;
    Vec<T> x;
    x.load(p);
    float f[E];
    x.to_float(f);
    const float2 *cs = tab + static_cast<int64_t>(pos) * (D / 2) + vi * (E / 2);
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
        const float2 c = cs[j];
        const double a = f[2 * j], b = f[2 * j + 1];
        f[2 * j] = static_cast<float>(a * c.x + b * static_cast<double>(c.y));
        f[2 * j + 1] = static_cast<float>(b * c.x - a * static_cast<double>(c.y));
    }
    Vec<T> y;
    y.from_float(f);
    y.store(p);
}

template <typename T, int D>
hipError_t launch_rope_backward_typed(void *grad, const int32_t *positions, int n_tokens, int n_heads,
                                      const float *freqs, int max_pos, hipStream_t s) {
    constexpr int VPR = D / Vec<T>::N;
    const int64_t total = static_cast<int64_t>(n_tokens) * n_heads * VPR;
    hipLaunchKernelGGL((rope_backward_kernel<T, D>), dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256),
                       0, s, static_cast<T *>(grad), positions, n_tokens, n_heads,
                       reinterpret_cast<const float2 *>(freqs), max_pos);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_rope_typed(const RopeArgs &a, hipStream_t s) {
    constexpr int VPR = D / Vec<T>::N;
    const int64_t total = static_cast<int64_t>(a.n_tokens) * (a.n_heads + 2 * a.pool.n_kv_heads) * VPR;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL((rope_kv_write_kernel<T, D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v),
                       a.positions, a.out_cache_loc, a.n_tokens, a.n_heads, a.pool.n_kv_heads,
                       reinterpret_cast<const float2 *>(a.freqs), a.max_pos,
                       static_cast<T *>(a.pool.k_layer), static_cast<T *>(a.pool.v_layer),
                       a.pool.pool_slots);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_table(float *freqs, int max_pos, int head_dim, double theta, hipStream_t s) {
    const int half = head_dim / 2;
    const int64_t total = static_cast<int64_t>(max_pos) * half;
    hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<float2 *>(freqs), max_pos, half, theta);
    return hipGetLastError();
}

hipError_t launch_rope_backward(void *grad, const int32_t *positions, int n_tokens, int n_heads, int head_dim,
                                int dtype, const float *freqs, int max_pos, hipStream_t s) {
    const bool bf = dtype == 1;
    if (head_dim == 128)
        return bf ? launch_rope_backward_typed<bf16_t, 128>(grad, positions, n_tokens, n_heads, freqs, max_pos, s)
                  : launch_rope_backward_typed<float, 128>(grad, positions, n_tokens, n_heads, freqs, max_pos, s);
    return bf ? launch_rope_backward_typed<bf16_t, 64>(grad, positions, n_tokens, n_heads, freqs, max_pos, s)
              : launch_rope_backward_typed<float, 64>(grad, positions, n_tokens, n_heads, freqs, max_pos, s);
}

hipError_t launch_rope_kv_write(const RopeArgs &a, hipStream_t s) {
    const bool bf = a.pool.dtype == 1;
    if (a.pool.head_dim == 128) return bf ? launch_rope_typed<bf16_t, 128>(a, s) : launch_rope_typed<float, 128>(a, s);
    return bf ? launch_rope_typed<bf16_t, 64>(a, s) : launch_rope_typed<float, 64>(a, s);
}

}  // namespace astr
