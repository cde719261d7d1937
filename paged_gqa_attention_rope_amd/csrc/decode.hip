// Split-K paged decode attention and its log-sum-exp merge.
//
// AstrAI docs/developer/internals.md, "KV Cache Mathematics":
// o_n = sum_j softmax(q_n k_j / sqrt(d_k)) v_j over a request's cached keys.
// docs/guides/inference.md, "KVCache System" and "Attention Backend": keys
// and values are read through req_to_token (one slot per token) at
// k/v_buffer[layer, slot, kv_head, :]; split-K writes partial outputs and
// max/log-sum partials that a second pass merges.
//
// Pass 1, one workgroup per (request b, KV head, split s): the split's KV
// positions are streamed once.  Each 16-byte slice of a KV row is read by one
// lane; a row (head_dim elements) is read by D/E consecutive lanes, so every
// wave-wide load is a run of whole 256-byte (bf16, D=128) row segments.  All
// G query heads of the KV head consume each row from registers, so the pool is
// read once per KV head, never once per query head.  Scores live in the log2
// domain (q is prescaled by sm_scale*log2(e)) and each lane group keeps an
// online softmax (running max, sum, output) per query head; U rows are loaded
// before any is used so that enough bytes are in flight to cover HBM latency.
// Lane groups are merged inside the wave by shuffles, waves through LDS.
//
// Pass 2, one wave per (b, query head): M = max_s lse_s,
// o = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M), over the request's
// ceil(L_b / C) splits.  When the batch has a single split the first pass
// writes the output directly and pass 2 is not launched.
#include "device.hpp"
#include "kernels.hpp"

namespace astr {
namespace {

constexpr float kLn2 = 0.693147180559945309f;

template <typename T, int D, int G>
struct DecodeCfg {
    static constexpr int E = Vec<T>::N;          // elements per lane per row
    static constexpr int LPR = D / E;            // lanes per KV row
    static constexpr int RPW = 64 / LPR;         // rows per wave-wide load
    static constexpr int WAVES = 4;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int NRG = THREADS / LPR;    // lane groups (row streams) per block
    static constexpr int U = 8;                  // rows in flight per lane group
};

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const T *__restrict__ q, T *__restrict__ out, float *__restrict__ o_part,
    float *__restrict__ lse_part, const T *__restrict__ k_layer, const T *__restrict__ v_layer,
    int64_t pool_slots, int n_kv, const int32_t *__restrict__ req_to_token, int num_reqs,
    int max_ctx_len, const int32_t *__restrict__ req_pool_indices,
    const int32_t *__restrict__ kv_indptr, int n_heads, int chunk, int n_splits, float scale_log2) {
    using C = DecodeCfg<T, D, G>;
    constexpr int E = C::E, LPR = C::LPR, NRG = C::NRG, U = C::U;

    const int kvh = blockIdx.x % n_kv;
    const int s = (blockIdx.x / n_kv) % n_splits;
    const int b = blockIdx.x / (n_kv * n_splits);
    const int req = req_pool_indices[b];
    const int L = request_len(kv_indptr, b, req, num_reqs, min(max_ctx_len, n_splits * chunk));
    const int start = s * chunk;
    if (start >= L && s > 0) return;              // empty split: the merge skips it
    const int end = min(start + chunk, L);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = tid % LPR;                    // which slice of the row
    const int rg = tid / LPR;                     // which row stream
    const int col = sub * E;

    float qf[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        Vec<T> x;
        x.load(q + (static_cast<int64_t>(b) * n_heads + kvh * G + g) * D + col);
        x.to_float(qf[g]);
#pragma unroll
        for (int e = 0; e < E; ++e) qf[g][e] *= scale_log2;
    }
    float m[G], l[G], acc[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
    }

    const int32_t *row = req_to_token + static_cast<int64_t>(req) * max_ctx_len;
    for (int t0 = start + rg; t0 < end; t0 += NRG * U) {
        Vec<T> kx[U], vx[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + u * NRG;
            int64_t slot = t < end ? row[t] : -1;
            ok[u] = slot >= 0 && slot < pool_slots;
            if (ok[u]) {
                const int64_t off = (slot * n_kv + kvh) * D + col;
                kx[u].load(k_layer + off);
                vx[u].load(v_layer + off);
            } else {
                kx[u].zero();
                vx[u].zero();
            }
        }
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[E];
            kx[u].to_float(kf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) d = fmaf(qf[g][e], kf[e], d);
#pragma unroll
                for (int o = 1; o < LPR; o <<= 1) d += __shfl_xor(d, o, 64);
                sc[u][g] = ok[u] ? d : -INFINITY;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mx = m[g];
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][g]);
            if (mx == -INFINITY) continue;
            const float alpha = exp2_sub(m[g], mx);
            l[g] *= alpha;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = exp2_sub(sc[u][g], mx);
                l[g] += p;
                float vf[E];
                vx[u].to_float(vf);
#pragma unroll
                for (int e = 0; e < E; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
            }
            m[g] = mx;
        }
    }

    // merge the row streams of this wave (lanes LPR, 2*LPR, ... apart)
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mo = __shfl_xor(m[g], o, 64);
            const float lo = __shfl_xor(l[g], o, 64);
            const float mx = fmaxf(m[g], mo);
            const float a = exp2_sub(m[g], mx), c = exp2_sub(mo, mx);
            l[g] = l[g] * a + lo * c;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float ao = __shfl_xor(acc[g][e], o, 64);
                acc[g][e] = acc[g][e] * a + ao * c;
            }
            m[g] = mx;
        }
    }
    // merge the waves through LDS
    __shared__ float s_m[C::WAVES][G], s_l[C::WAVES][G];
    __shared__ float s_acc[C::WAVES][G][D];
    if (lane < LPR) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (lane == 0) {
                s_m[wave][g] = m[g];
                s_l[wave][g] = l[g];
            }
#pragma unroll
            for (int e = 0; e < E; ++e) s_acc[wave][g][col + e] = acc[g][e];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += C::THREADS) {
        const int g = idx / D, d = idx % D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < C::WAVES; ++w) mx = fmaxf(mx, s_m[w][g]);
        float lsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < C::WAVES; ++w) {
            const float a = exp2_sub(s_m[w][g], mx);
            lsum += s_l[w][g] * a;
            o += s_acc[w][g][d] * a;
        }
        const int h = kvh * G + g;
        const float res = lsum > 0.f ? o / lsum : 0.f;
        if (n_splits == 1) {
            store_scalar<T>(out + (static_cast<int64_t>(b) * n_heads + h) * D + d, res);
        } else {
            const int64_t ps = (static_cast<int64_t>(b) * n_heads + h) * n_splits + s;
            o_part[ps * D + d] = res;
            if (d == 0) lse_part[ps] = lsum > 0.f ? (mx + __log2f(lsum)) * kLn2 : -INFINITY;
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float *__restrict__ o_part, const float *__restrict__ lse_part, T *__restrict__ out,
    const int32_t *__restrict__ kv_indptr, const int32_t *__restrict__ req_pool_indices,
    int num_reqs, int max_ctx_len, int batch, int n_heads, int chunk, int n_splits) {
    constexpr int PER = D / 64;
    const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (bh >= batch * n_heads) return;
    const int b = bh / n_heads;
    const int L = request_len(kv_indptr, b, req_pool_indices[b], num_reqs,
                              min(max_ctx_len, n_splits * chunk));
    const int ns = min((L + chunk - 1) / chunk, n_splits);
    const float *lse = lse_part + static_cast<int64_t>(bh) * n_splits;
    const float *op = o_part + static_cast<int64_t>(bh) * n_splits * D;
    float mx = -INFINITY;
    for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, lse[s]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float acc[PER] = {};
    float wsum = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float w = lse[s] == -INFINITY ? 0.f : __expf(lse[s] - mx);
        wsum += w;
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] = fmaf(w, op[static_cast<int64_t>(s) * D + lane + 64 * j], acc[j]);
    }
    T *dst = out + static_cast<int64_t>(bh) * D;
#pragma unroll
    for (int j = 0; j < PER; ++j) store_scalar<T>(dst + lane + 64 * j, wsum > 0.f ? acc[j] / wsum : 0.f);
}

template <typename T, int D, int G>
hipError_t launch_decode_typed(const DecodeArgs &a, hipStream_t s) {
    const int n_kv = a.pool.n_kv_heads;
    const int64_t blocks = static_cast<int64_t>(a.batch) * a.n_splits * n_kv;
    hipLaunchKernelGGL((decode_split_kernel<T, D, G>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const T *>(a.q), static_cast<T *>(a.out), a.o_part, a.lse_part,
                       static_cast<const T *>(a.pool.k_layer), static_cast<const T *>(a.pool.v_layer),
                       a.pool.pool_slots, n_kv, a.req_to_token, a.num_reqs, a.max_ctx_len,
                       a.req_pool_indices, a.kv_indptr, a.n_heads, a.split_chunk, a.n_splits,
                       a.scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_splits == 1) return e;
    const int64_t mblocks = (static_cast<int64_t>(a.batch) * a.n_heads + 3) / 4;
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(static_cast<unsigned>(mblocks)), dim3(256), 0, s,
                       a.o_part, a.lse_part, static_cast<T *>(a.out), a.kv_indptr,
                       a.req_pool_indices, a.num_reqs, a.max_ctx_len, a.batch, a.n_heads,
                       a.split_chunk, a.n_splits);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_g(const DecodeArgs &a, hipStream_t s) {
    switch (a.n_heads / a.pool.n_kv_heads) {
        case 1: return launch_decode_typed<T, D, 1>(a, s);
        case 2: return launch_decode_typed<T, D, 2>(a, s);
        case 4: return launch_decode_typed<T, D, 4>(a, s);
        case 6: return launch_decode_typed<T, D, 6>(a, s);
        case 8: return launch_decode_typed<T, D, 8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    const bool bf = a.pool.dtype == 1;
    if (a.pool.head_dim == 128) return bf ? launch_decode_g<bf16_t, 128>(a, s) : launch_decode_g<float, 128>(a, s);
    return bf ? launch_decode_g<bf16_t, 64>(a, s) : launch_decode_g<float, 64>(a, s);
}

}  // namespace astr
