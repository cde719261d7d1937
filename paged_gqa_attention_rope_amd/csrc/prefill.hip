// Ragged causal prefill attention over the paged pool.
//
// AstrAI docs/guides/inference.md, "KVCache System" and "Attention Backend":
// a ragged batch is addressed by qo_indptr (query rows) and kv_indptr (KV
// lengths); the query-tile maps q_tile_to_batch / q_tile_to_index assign each
// tile of q_tile rows to its request; keys and values are read from the flat
// pool through req_to_token.  docs/developer/internals.md, "Autoregression &
// Causal Masking": position i attends keys j <= i; with a cached prefix of
// p = L - e positions, query i of the request sits at position p + i.
//
// Two kernels:
//  * prefill_mfma (bf16): one workgroup per (query tile, KV head) holds the
//    tile's 64 rows for all G query heads of that KV head (2G waves, 32 rows
//    of one head each), so every K/V tile staged in LDS serves 64*G rows.
//    QK^T and PV run on the gfx950 bf16 matrix cores
//    (v_mfma_f32_16x16x32_bf16).  The product is formed transposed,
//    S^T = K Q^T, so that a lane's accumulator registers hold one query row's
//    scores for 8 keys -- exactly the B-operand slice the PV product
//    O^T = V^T P^T needs, with the key order of the reduction chosen to match.
//    P never leaves registers.  V is stored transposed in LDS for the A
//    operand; rows are padded by 16 bytes against bank conflicts.  Online
//    softmax in the log2 domain, fp32 accumulators; P is rounded to bf16 for
//    the PV product.  Only tiles that cross the causal diagonal are masked.
//  * prefill_generic (float32):
//    one workgroup per (query tile, query head), 4 lanes per query row,
//    K/V tiles of 32 keys staged in LDS as float32, online softmax per key.
#include "device.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace astr {
namespace {

// Row range and KV extent of query tile `t`; false when the tile is empty or
// its metadata is inconsistent (then the tile is skipped).
struct TileInfo {
    int b, req, q0, e, L, p, row0, rows, kv_end;
};

__device__ __forceinline__ bool tile_info(int t, const int32_t *q_tile_to_batch,
                                          const int32_t *q_tile_to_index, const int32_t *qo_indptr,
                                          const int32_t *kv_indptr, const int32_t *req_pool_indices,
                                          int batch, int num_reqs, int max_ctx_len, int total_q,
                                          int q_tile, TileInfo &ti) {
    ti.b = q_tile_to_batch[t];
    if (ti.b < 0 || ti.b >= batch) return false;
    const int idx = q_tile_to_index[t];
    ti.req = req_pool_indices[ti.b];
    ti.q0 = qo_indptr[ti.b];
    ti.e = qo_indptr[ti.b + 1] - ti.q0;
    ti.L = request_len(kv_indptr, ti.b, ti.req, num_reqs, max_ctx_len);
    ti.p = ti.L - ti.e;
    ti.row0 = idx * q_tile;
    if (idx < 0 || ti.e <= 0 || ti.p < 0 || ti.row0 >= ti.e) return false;
    if (ti.q0 < 0 || ti.q0 > total_q - ti.e) return false;
    ti.rows = min(q_tile, ti.e - ti.row0);
    ti.kv_end = ti.p + ti.row0 + ti.rows;       // keys seen by the tile's last row
    return true;
}

// ---------------------------------------------------------------------------
// generic kernel
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_generic_kernel(
    const T *__restrict__ q, T *__restrict__ out, const T *__restrict__ k_layer,
    const T *__restrict__ v_layer, int64_t pool_slots, int n_kv,
    const int32_t *__restrict__ req_to_token, int num_reqs, int max_ctx_len,
    const int32_t *__restrict__ req_pool_indices, const int32_t *__restrict__ qo_indptr,
    const int32_t *__restrict__ kv_indptr, const int32_t *__restrict__ q_tile_to_batch,
    const int32_t *__restrict__ q_tile_to_index, int batch, int total_q, int n_heads,
    float scale_log2) {
    constexpr int TQ = 64, LPQ = 4, DL = D / LPQ, TK = 32;
    constexpr int E = Vec<T>::N, SL = D / E;      // 16-byte slices per row
    TileInfo ti;
    if (!tile_info(blockIdx.x, q_tile_to_batch, q_tile_to_index, qo_indptr, kv_indptr,
                   req_pool_indices, batch, num_reqs, max_ctx_len, total_q, TQ, ti))
        return;
    const int h = blockIdx.y;
    const int kvh = h / (n_heads / n_kv);
    const int tid = threadIdx.x;
    const int r = tid / LPQ, part = tid % LPQ;
    const int i = ti.row0 + r;                     // request-local query index
    const bool valid = r < ti.rows;

    float qv[DL];
    {
        const T *src = q + (static_cast<int64_t>(ti.q0 + (valid ? i : ti.row0)) * n_heads + h) * D + part * DL;
#pragma unroll
        for (int c = 0; c < DL; c += E) {
            Vec<T> x;
            x.load(src + c);
            float f[E];
            x.to_float(f);
#pragma unroll
            for (int e = 0; e < E; ++e) qv[c + e] = f[e] * scale_log2;
        }
    }
    float m = -INFINITY, l = 0.f, acc[DL];
#pragma unroll
    for (int d = 0; d < DL; ++d) acc[d] = 0.f;

    __shared__ float sK[TK][D + 4];
    __shared__ float sV[TK][D + 4];
    __shared__ int sOk[TK];
    const int32_t *row = req_to_token + static_cast<int64_t>(ti.req) * max_ctx_len;
    for (int kt = 0; kt < ti.kv_end; kt += TK) {
        for (int sidx = tid; sidx < TK * SL; sidx += 256) {
            const int kr = sidx / SL, c = (sidx % SL) * E;
            const int j = kt + kr;
            const int64_t slot = j < ti.kv_end ? row[j] : -1;
            const bool ok = slot >= 0 && slot < pool_slots;
            Vec<T> kx, vx;
            if (ok) {
                kx.load(k_layer + (slot * n_kv + kvh) * D + c);
                vx.load(v_layer + (slot * n_kv + kvh) * D + c);
            } else {
                kx.zero();
                vx.zero();
            }
            float fk[E], fv[E];
            kx.to_float(fk);
            vx.to_float(fv);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                sK[kr][c + e] = fk[e];
                sV[kr][c + e] = fv[e];
            }
            if (c == 0) sOk[kr] = ok;
        }
        __syncthreads();
        const int nk = min(TK, ti.kv_end - kt);
        for (int jj = 0; jj < nk; ++jj) {
            float s = 0.f;
#pragma unroll
            for (int d = 0; d < DL; ++d) s = fmaf(qv[d], sK[jj][part * DL + d], s);
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            const bool vis = sOk[jj] && (kt + jj <= ti.p + i);
            if (vis) {
                const float mn = fmaxf(m, s);
                const float a = exp2_sub(m, mn);
                const float pj = exp2f(s - mn);
                l = l * a + pj;
#pragma unroll
                for (int d = 0; d < DL; ++d) acc[d] = fmaf(pj, sV[jj][part * DL + d], acc[d] * a);
                m = mn;
            }
        }
        __syncthreads();
    }
    if (!valid) return;
    T *dst = out + (static_cast<int64_t>(ti.q0 + i) * n_heads + h) * D + part * DL;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < DL; c += E) {
        float f[E];
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = acc[c + e] * inv;
        Vec<T> y;
        y.from_float(f);
        y.store(dst + c);
    }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
template <int D, int G>
struct MfmaCfg {
    static constexpr int TQ = 64;            // query rows per tile
    static constexpr int RB = 2;             // 16-row blocks per wave (32 rows)
    static constexpr int WAVES = 2 * G;      // 2 waves per query head
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TK = 64;            // keys per LDS tile
    static constexpr int KB = TK / 16;       // 16-key blocks per tile
    static constexpr int KS = D / 32;        // k-steps of the QK^T product
    static constexpr int DB = D / 16;        // 16-wide d blocks of the output
    static constexpr int LDK = D + 8;        // padded K row (bf16 elements)
    static constexpr int LDV = TK + 8;       // padded V^T row (bf16 elements)
};

template <int D, int G>
__global__ __launch_bounds__((MfmaCfg<D, G>::THREADS)) void prefill_mfma_kernel(
    const uint16_t *__restrict__ q, uint16_t *__restrict__ out, const uint16_t *__restrict__ k_layer,
    const uint16_t *__restrict__ v_layer, int64_t pool_slots, int n_kv,
    const int32_t *__restrict__ req_to_token, int num_reqs, int max_ctx_len,
    const int32_t *__restrict__ req_pool_indices, const int32_t *__restrict__ qo_indptr,
    const int32_t *__restrict__ kv_indptr, const int32_t *__restrict__ q_tile_to_batch,
    const int32_t *__restrict__ q_tile_to_index, int batch, int total_q, int n_heads,
    float scale_log2) {
    using C = MfmaCfg<D, G>;
    constexpr int TQ = C::TQ, RB = C::RB, TK = C::TK, KB = C::KB, KS = C::KS, DB = C::DB;
    constexpr int LDK = C::LDK, LDV = C::LDV;
    constexpr int SL = D / 8;                    // 16-byte slices per K/V row

    TileInfo ti;
    if (!tile_info(blockIdx.x, q_tile_to_batch, q_tile_to_index, qo_indptr, kv_indptr,
                   req_pool_indices, batch, num_reqs, max_ctx_len, total_q, TQ, ti))
        return;
    const int kvh = blockIdx.y;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int h = kvh * G + (wave >> 1);
    const int wrow0 = (wave & 1) * (16 * RB);    // first tile row of this wave
    const int ln = lane & 15, lg = lane >> 4;    // MFMA column / lane group

    __shared__ __attribute__((aligned(16))) uint16_t sK[TK * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[D * LDV];
    __shared__ int sOk[TK];

    // Q^T operand (B of S^T = K Q^T): lane holds row (ln) of each row block,
    // d = 32*ks + 8*lg .. +7.  Rows past the tile end read row 0 (results unused).
    Frag8 qf[RB][KS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int r = wrow0 + 16 * rb + ln;
        if (r >= ti.rows) r = 0;
        const uint16_t *src = q + (static_cast<int64_t>(ti.q0 + ti.row0 + r) * n_heads + h) * D + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[rb][ks].u = *reinterpret_cast<const uint4 *>(src + 32 * ks);
    }
    f32x4_t o[RB][DB];
    float m[RB], lsum[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m[rb] = -INFINITY;
        lsum[rb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // this wave's last row and the keys it needs
    const int wrows = min(16 * RB, ti.rows - wrow0);
    const int w_kv_end = wrows > 0 ? ti.p + ti.row0 + wrow0 + wrows : 0;

    const int32_t *trow = req_to_token + static_cast<int64_t>(ti.req) * max_ctx_len;
    for (int kt = 0; kt < ti.kv_end; kt += TK) {
        // stage K (row-major) and V^T (transposed) for keys kt .. kt+TK-1
        for (int sidx = tid; sidx < TK * SL; sidx += C::THREADS) {
            const int kr = sidx / SL, c = (sidx % SL) * 8;
            const int j = kt + kr;
            const int64_t slot = j < ti.kv_end ? trow[j] : -1;
            const bool ok = slot >= 0 && slot < pool_slots;
            uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
            if (ok) {
                kx = *reinterpret_cast<const uint4 *>(k_layer + (slot * n_kv + kvh) * D + c);
                vx = *reinterpret_cast<const uint4 *>(v_layer + (slot * n_kv + kvh) * D + c);
            }
            *reinterpret_cast<uint4 *>(&sK[kr * LDK + c]) = kx;
            const uint32_t vw[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sVt[(c + 2 * e) * LDV + kr] = static_cast<uint16_t>(vw[e] & 0xffffu);
                sVt[(c + 2 * e + 1) * LDV + kr] = static_cast<uint16_t>(vw[e] >> 16);
            }
            if (c == 0) sOk[kr] = ok;
        }
        __syncthreads();
        if (kt < w_kv_end) {
            // S^T[key][row] for KB key blocks x RB row blocks
            f32x4_t s[RB][KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) s[rb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    Frag8 kf;
                    kf.u = *reinterpret_cast<const uint4 *>(&sK[(16 * kb + ln) * LDK + 32 * ks + 8 * lg]);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) s[rb][kb] = mfma16(kf, qf[rb][ks], s[rb][kb]);
                }
            }
            // scale, mask, online softmax; lane holds keys 16*kb + 4*lg + r of row ln
            const bool diag = kt + TK - 1 > ti.p + ti.row0 + wrow0;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int qi = ti.row0 + wrow0 + 16 * rb + ln;    // request-local query index
                float mx = m[rb];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int kl = 16 * kb + 4 * lg + r;
                        float x = s[rb][kb][r] * scale_log2;
                        if (!sOk[kl] || (diag && kt + kl > ti.p + qi)) x = -INFINITY;
                        s[rb][kb][r] = x;
                        mx = fmaxf(mx, x);
                    }
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float alpha = exp2_sub(m[rb], mx);
                m[rb] = mx;
                float ps = 0.f;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float pv = exp2_sub(s[rb][kb][r], mx);
                        s[rb][kb][r] = pv;
                        ps += pv;
                    }
                }
                lsum[rb] = lsum[rb] * alpha + ps;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[rb][db][r] *= alpha;
                }
            }
            // O^T += V^T P^T; reduction slot 8*lg + r <-> key 32*ks2 + 4*lg + r,
            // slot 8*lg + 4 + r <-> key 32*ks2 + 16 + 4*lg + r
#pragma unroll
            for (int ks2 = 0; ks2 < TK / 32; ++ks2) {
                Frag8 pf[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const f32x4_t a = s[rb][2 * ks2], b = s[rb][2 * ks2 + 1];
                    pf[rb].w[0] = pack_bf16x2(a[0], a[1]);
                    pf[rb].w[1] = pack_bf16x2(a[2], a[3]);
                    pf[rb].w[2] = pack_bf16x2(b[0], b[1]);
                    pf[rb].w[3] = pack_bf16x2(b[2], b[3]);
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint16_t *vrow = &sVt[(16 * db + ln) * LDV + 32 * ks2 + 4 * lg];
                    Frag8 vf;
                    const uint2 lo = *reinterpret_cast<const uint2 *>(vrow);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 16);
                    vf.w[0] = lo.x;
                    vf.w[1] = lo.y;
                    vf.w[2] = hi.x;
                    vf.w[3] = hi.y;
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma16(vf, pf[rb], o[rb][db]);
                }
            }
        }
        __syncthreads();
    }
    // finish: row sums across the 4 lane groups, normalise, store
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float ls = lsum[rb];
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        const int r = wrow0 + 16 * rb + ln;
        if (r >= ti.rows) continue;
        const float inv = ls > 0.f ? 1.f / ls : 0.f;
        uint16_t *dst = out + (static_cast<int64_t>(ti.q0 + ti.row0 + r) * n_heads + h) * D + 4 * lg;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            uint2 w;
            w.x = pack_bf16x2(o[rb][db][0] * inv, o[rb][db][1] * inv);
            w.y = pack_bf16x2(o[rb][db][2] * inv, o[rb][db][3] * inv);
            *reinterpret_cast<uint2 *>(dst + 16 * db) = w;
        }
    }
}

template <typename T, int D>
hipError_t launch_generic(const PrefillArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((prefill_generic_kernel<T, D>), dim3(a.num_q_tiles, a.n_heads), dim3(256), 0, s,
                       static_cast<const T *>(a.q), static_cast<T *>(a.out),
                       static_cast<const T *>(a.pool.k_layer), static_cast<const T *>(a.pool.v_layer),
                       a.pool.pool_slots, a.pool.n_kv_heads, a.req_to_token, a.num_reqs, a.max_ctx_len,
                       a.req_pool_indices, a.qo_indptr, a.kv_indptr, a.q_tile_to_batch,
                       a.q_tile_to_index, a.batch, a.total_q, a.n_heads, a.scale_log2);
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_mfma(const PrefillArgs &a, hipStream_t s) {
    using C = MfmaCfg<D, G>;
    hipLaunchKernelGGL((prefill_mfma_kernel<D, G>), dim3(a.num_q_tiles, a.pool.n_kv_heads), dim3(C::THREADS),
                       0, s, static_cast<const uint16_t *>(a.q), static_cast<uint16_t *>(a.out),
                       static_cast<const uint16_t *>(a.pool.k_layer),
                       static_cast<const uint16_t *>(a.pool.v_layer), a.pool.pool_slots,
                       a.pool.n_kv_heads, a.req_to_token, a.num_reqs, a.max_ctx_len, a.req_pool_indices,
                       a.qo_indptr, a.kv_indptr, a.q_tile_to_batch, a.q_tile_to_index, a.batch,
                       a.total_q, a.n_heads, a.scale_log2);
    return hipGetLastError();
}

template <int D>
hipError_t launch_mfma_g(const PrefillArgs &a, hipStream_t s) {
    switch (a.n_heads / a.pool.n_kv_heads) {
        case 1: return launch_mfma<D, 1>(a, s);
        case 2: return launch_mfma<D, 2>(a, s);
        case 4: return launch_mfma<D, 4>(a, s);
        case 6: return launch_mfma<D, 6>(a, s);
        case 8: return launch_mfma<D, 8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
    if (a.num_q_tiles == 0) return hipSuccess;
    if (a.pool.dtype == 1)
        return a.pool.head_dim == 128 ? launch_mfma_g<128>(a, s) : launch_mfma_g<64>(a, s);
    return a.pool.head_dim == 128 ? launch_generic<float, 128>(a, s) : launch_generic<float, 64>(a, s);
}

}  // namespace astr
