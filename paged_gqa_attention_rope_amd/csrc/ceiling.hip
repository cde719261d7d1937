// Attainable-rate probes: a plain streaming read of a device buffer and a
// loop of independent bf16 matrix-core products.  They are not part of the
// attention path; the benchmark runs them beside it so that each kernel's
// rate can be read against what the chip delivers for the same kind of work
// (HBM reads, v_mfma_f32_16x16x32_bf16), as well as against the nominal
// peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace astr {
namespace {

// Grid-stride read of n16 16-byte chunks; every lane folds what it read into
// an xor so that no load can be dropped, and one lane per workgroup stores
// the workgroup's fold.
template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ buf, uint64_t n16,
                                                          uint32_t *__restrict__ sink) {
    uint32_t acc = 0;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    // eight independent loads in flight per lane
    constexpr int U = 8;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (NT) v[u] = load_nt16(buf + i + u * stride);
            else v[u] = buf[i + u * stride];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        uint4 v;
        if constexpr (NT) v = load_nt16(buf + i);
        else v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // fold the workgroup: lane 0 of each wave, then one store
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    __shared__ uint32_t w[4];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = w[0] ^ w[1] ^ w[2] ^ w[3];
}

// A bf16 pair with random signs and mantissas and magnitudes in about
// [2^-7, 2^2): operands whose bits toggle like real activations do (the
// matrix cores draw more power, and the clock drops further, than with
// constant or mostly-zero operands).
__device__ __forceinline__ uint32_t random_bf16_pair(uint32_t x) {
    x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
    const uint32_t lo = (x & 0x807fu) | ((120u + (x >> 8) % 9u) << 7);
    const uint32_t hi = ((x >> 16) & 0x807fu) | ((120u + (x >> 24) % 9u) << 7);
    return lo | (hi << 16);
}

// Each wave keeps 8 independent accumulators and issues 8 products per
// iteration from operands held in registers.  The accumulators start from
// distinct values: started from one shared constant, the compiler rotates
// them through overlapping registers, which chains the products.  One store
// per lane at the end.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float *__restrict__ sink) {
    Frag8 a, b;
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a.w[e] = random_bf16_pair(8u * t + e);
        b.w[e] = random_bf16_pair(8u * t + 4u + e);
    }
    f32x4_t acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float x = static_cast<float>(threadIdx.x * 8 + k);
        acc[k] = f32x4_t{x, x + 1.f, x + 2.f, x + 3.f};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = mfma16(a, b, acc[k]);
    }
    f32x4_t s = acc[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) s += acc[k];
    sink[static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

}  // namespace

hipError_t launch_ceiling_stream_read(const void *buf, uint64_t bytes, int workgroups, bool nontemporal,
                                      uint32_t *sink, hipStream_t s) {
    const uint64_t n16 = bytes / 16;
    if (nontemporal)
        hipLaunchKernelGGL(stream_read_kernel<true>, dim3(workgroups), dim3(256), 0, s,
                           static_cast<const uint4 *>(buf), n16, sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<false>, dim3(workgroups), dim3(256), 0, s,
                           static_cast<const uint4 *>(buf), n16, sink);
    return hipGetLastError();
}

hipError_t launch_ceiling_mfma_loop(int workgroups, int iters, float *sink, hipStream_t s) {
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, s, iters, sink);
    return hipGetLastError();
}

}  // namespace astr
