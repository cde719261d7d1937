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
// acc *= alpha with each result tied to its own register: on the rarely
// taken rescale path the accumulators keep their registers, so the branch
// join needs no copies on the common path.
__device__ __forceinline__ void scale_in_place(f32x4_t &acc, float alpha) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float x = acc[r];
        asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x) : "v"(alpha));
        acc[r] = x;
    }
}

constexpr int kXcds = 8;        // accelerator dies (XCDs) of an MI355X, each with its own L2

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
    static constexpr int TQ = 64;                    // query rows per tile
    static constexpr int HW = G == 1 ? 1 : 2;        // query heads per wave
    static constexpr int GROUPS = G / HW;            // head groups: grid z
    static constexpr int WAVES = 4;                  // 4 row blocks of 16
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TK = 64;                    // keys per LDS tile
    static constexpr int KS = D / 32;                // k-steps of the QK^T product
    static constexpr int DB = D / 16;                // 16-wide d blocks of the output
    // padded K/V row (bf16 elements): a 32-byte pad puts consecutive rows 8
    // banks apart, so the 4 rows x 32 bytes a 16-lane group touches in one
    // transposing read, and the 16 rows of a 128-bit operand read, spread evenly
    static constexpr int LDK = D + 16;
    static constexpr int SL = D / 8;                 // 16-byte slices per row
    static constexpr int NLD = TK * SL / THREADS;    // K (and V) loads per thread per tile
    static constexpr int BUF = 2 * TK * LDK;         // K + V tile, bf16 elements
    static_assert(G % HW == 0 && NLD >= 1 && (TK * SL) % THREADS == 0, "tiling");
};

// One workgroup per (query tile, KV head, head group of HW query heads).
// Wave w owns query rows 16w .. 16w+15 of the tile for the HW heads, so every K
// and V operand read from LDS feeds HW matrix-core products, and holds their
// Q^T operands and O^T accumulators in registers.  K/V tiles of 64 keys are
// gathered (whole 256-byte rows, non-temporal) into registers one tile ahead
// and written to the other half of a double-buffered LDS tile; slot indices
// are fetched two tiles ahead.  Per 32 keys: S^T = K Q^T, online softmax in
// the log2 domain with the running max raised only when a row's max grows by
// more than 8 (exact: the same stale max is used for numerator and
// denominator, and probabilities stay below 2^8), then O^T += V^T P^T with P
// straight from the accumulators and V^T from the LDS transpose read.
template <int D, int G>
__global__ __launch_bounds__((MfmaCfg<D, G>::THREADS), 2) void prefill_mfma_kernel(
    const uint16_t *__restrict__ q, uint16_t *__restrict__ out, const uint16_t *__restrict__ k_layer,
    const uint16_t *__restrict__ v_layer, int64_t pool_slots, int n_kv,
    const int32_t *__restrict__ req_to_token, int num_reqs, int max_ctx_len,
    const int32_t *__restrict__ req_pool_indices, const int32_t *__restrict__ qo_indptr,
    const int32_t *__restrict__ kv_indptr, const int32_t *__restrict__ q_tile_to_batch,
    const int32_t *__restrict__ q_tile_to_index, int batch, int total_q, int n_heads,
    int num_q_tiles, float scale_log2) {
    using C = MfmaCfg<D, G>;
    constexpr int TQ = C::TQ, HW = C::HW, TK = C::TK, KS = C::KS, DB = C::DB, LDK = C::LDK;
    constexpr int SL = C::SL, NLD = C::NLD;
    constexpr float kLazy = 8.f;                     // log2-domain slack before a rescale

    // Workgroups are handed to the 8 XCDs round-robin (id % 8).  The tiles
    // arrive heaviest first, so give XCD c the tiles of rank c, c+8, c+16, ...
    // (every die gets a balanced, heaviest-first share), and keep all KV heads
    // and head groups of one tile -- which read the same K/V rows -- on the
    // die that owns the tile, sharing its L2.  The grid is padded to a
    // multiple of 8 tiles; padding blocks exit at once.
    const int units_per_tile = n_kv * C::GROUPS;
    const int xcd = blockIdx.x % kXcds, k_in = blockIdx.x / kXcds;
    const int tile = kXcds * (k_in / units_per_tile) + xcd;
    if (tile >= num_q_tiles) return;
    const int u = k_in % units_per_tile;
    const int kvh = u / C::GROUPS;
    const int grp = u % C::GROUPS;
    TileInfo ti;
    if (!tile_info(tile, q_tile_to_batch, q_tile_to_index, qo_indptr, kv_indptr,
                   req_pool_indices, batch, num_reqs, max_ctx_len, total_q, TQ, ti))
        return;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, j = lane & 15;
    const int r0 = 16 * wave;                        // first tile row of this wave
    const int h0 = kvh * G + grp * HW;               // first query head of this wave
    const int qpos0 = ti.p + ti.row0 + r0;           // position of the wave's first row
    const int qpos = qpos0 + j;                      // position of this lane's row

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];
    __shared__ uint8_t sOk[2][TK];

    // Q^T operands: lane (g, j) holds row r0 + j, d = 32ks + 8g .. +7 of each head
    Frag8 qf[HW][KS];
    {
        int r = r0 + j;
        if (r >= ti.rows) r = 0;                     // rows past the tile end: results unused
        const uint16_t *src = q + (static_cast<int64_t>(ti.q0 + ti.row0 + r) * n_heads + h0) * D + 8 * g;
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[hh][ks].u = *reinterpret_cast<const uint4 *>(src + hh * D + 32 * ks);
        }
    }
    f32x4_t o[HW][DB], osum[HW];                    // osum: row sums of P (all 4 entries equal)
    float m[HW];
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
        m[hh] = -INFINITY;
        osum[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < DB; ++db) o[hh][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    Frag8 ones;                                      // bf16 1.0 in every reduction slot
    ones.u = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);

    // gather assignment: load i of this thread covers key (tid + THREADS*i) / SL
    // of the tile, 16-byte slice (tid + THREADS*i) % SL, for both K and V
    const int32_t *trow = req_to_token + static_cast<int64_t>(ti.req) * max_ctx_len;
    // Loads are unconditional (an out-of-range key or slot reads row 0 of the
    // table or pool instead) so that no branch joins force an early wait on the
    // prefetch; invalid rows are zeroed when staged and masked by sOk.
    auto slots_of = [&](int kt, int32_t (&sl)[NLD]) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int key = kt + (tid + C::THREADS * i) / SL;
            const int32_t v = trow[min(key, ti.kv_end - 1)];
            sl[i] = key < ti.kv_end ? v : -1;
        }
    };
    const int row_elems = n_kv * D;                  // pool elements per slot
    auto gather = [&](const int32_t (&sl)[NLD], uint4 (&kx)[NLD], uint4 (&vx)[NLD]) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int32_t slot = sl[i] >= 0 && sl[i] < pool_slots ? sl[i] : 0;
            const int64_t off = static_cast<int64_t>(slot) * row_elems +
                                (kvh * D + 8 * ((tid + C::THREADS * i) % SL));
            // cached loads: every tile of the request reads these rows again
            kx[i] = *reinterpret_cast<const uint4 *>(k_layer + off);
            vx[i] = *reinterpret_cast<const uint4 *>(v_layer + off);
        }
    };
    auto stage = [&](int buf, const int32_t (&sl)[NLD], const uint4 (&kx)[NLD], const uint4 (&vx)[NLD]) {
        uint16_t *sK = smem + buf * C::BUF;
        uint16_t *sV = sK + TK * LDK;
        bool all_ok = true;
#pragma unroll
        for (int i = 0; i < NLD; ++i) all_ok = all_ok && sl[i] >= 0 && sl[i] < pool_slots;
        if (__all(all_ok)) {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int idx = tid + C::THREADS * i;
                const int key = idx / SL, c = (idx % SL) * 8;
                *reinterpret_cast<uint4 *>(sK + key * LDK + c) = kx[i];
                *reinterpret_cast<uint4 *>(sV + key * LDK + c) = vx[i];
                if (c == 0) sOk[buf][key] = 1;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int idx = tid + C::THREADS * i;
                const int key = idx / SL, c = (idx % SL) * 8;
                const bool ok = sl[i] >= 0 && sl[i] < pool_slots;
                const uint32_t keep = ok ? 0xffffffffu : 0u;  // value select, no branch
                uint4 kv = kx[i], vv = vx[i];
                kv.x &= keep; kv.y &= keep; kv.z &= keep; kv.w &= keep;
                vv.x &= keep; vv.y &= keep; vv.z &= keep; vv.w &= keep;
                *reinterpret_cast<uint4 *>(sK + key * LDK + c) = kv;
                *reinterpret_cast<uint4 *>(sV + key * LDK + c) = vv;
                if (c == 0) sOk[buf][key] = ok;
            }
        }
    };

    int32_t sl_cur[NLD], sl_nxt[NLD];
    uint4 kx[NLD], vx[NLD];
    slots_of(0, sl_cur);
    slots_of(TK, sl_nxt);
    gather(sl_cur, kx, vx);
    stage(0, sl_cur, kx, vx);
    __syncthreads();

    const int w_last = min(r0 + 15, ti.rows - 1);    // the wave's last valid row
    const int w_kv_end = w_last >= r0 ? ti.p + ti.row0 + w_last + 1 : 0;
    for (int kt = 0, it = 0; kt < ti.kv_end; kt += TK, ++it) {
        const int buf = it & 1;
        const bool has_next = kt + TK < ti.kv_end;
        int32_t sl_new[NLD];
        if (has_next) {
            // slot indices of tile it+2 first: loads retire in order, so anything
            // that waits for them must not also wait for the K/V prefetch
            slots_of(kt + 2 * TK, sl_new);
            gather(sl_nxt, kx, vx);                  // tile it+1, in flight during compute
        }
        const uint64_t okm = __ballot(sOk[buf][lane] != 0);
        const uint16_t *sK = smem + buf * C::BUF;
        const uint16_t *sV = sK + TK * LDK;
#pragma unroll 1   // one register assignment for the accumulators (no rotation copies)
        for (int sub = 0; sub < TK / 32; ++sub) {
            const int kb0 = kt + 32 * sub;           // first key of this 32-key step
            // a step past the wave's last visible key is fully masked below and
            // adds nothing (no early exit: that would split the accumulators'
            // live ranges across a branch join)
            const bool diag = kb0 + 31 > qpos0;
            f32x4_t sc[HW][2];
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) {
                sc[hh][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                sc[hh][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    Frag8 kf;
                    kf.u = *reinterpret_cast<const uint4 *>(sK + (32 * sub + 16 * kb + j) * LDK + 32 * ks + 8 * g);
#pragma unroll
                    for (int hh = 0; hh < HW; ++hh) sc[hh][kb] = mfma16(kf, qf[hh][ks], sc[hh][kb]);
                }
            }
            // keys of this lane: kb0 + 16kb + 4g + r; row: qpos.  Masking is needed
            // only where the step crosses the causal diagonal or a slot is missing.
            const uint32_t okw = static_cast<uint32_t>(okm >> (32 * sub));
            if (diag || okw != 0xffffffffu) {
#pragma unroll
                for (int hh = 0; hh < HW; ++hh) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int k = 16 * kb + 4 * g + r;
                            if (!((okw >> k) & 1u) || kb0 + k > qpos) sc[hh][kb][r] = -INFINITY;
                        }
                    }
                }
            }
            // running max per head; the accumulators are rescaled only when some
            // row's max grew by more than kLazy (one wave-uniform branch)
            float mnew[HW];
            bool need_any = false;
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) {
                float mxr = fmaxf(fmaxf(fmaxf(sc[hh][0][0], sc[hh][0][1]), fmaxf(sc[hh][0][2], sc[hh][0][3])),
                                  fmaxf(fmaxf(sc[hh][1][0], sc[hh][1][1]), fmaxf(sc[hh][1][2], sc[hh][1][3])));
                const float mx = max_over_groups(mxr) * scale_log2;   // scale > 0 keeps the order
                const bool need = mx > m[hh] + kLazy;
                mnew[hh] = need ? mx : m[hh];
                need_any = need_any || need;
            }
            if (__builtin_expect(__any(need_any), 0)) {
#pragma unroll
                for (int hh = 0; hh < HW; ++hh) {
                    const float alpha = exp2_sub(m[hh], mnew[hh]);   // 1 where m is unchanged
                    scale_in_place(osum[hh], alpha);
#pragma unroll
                    for (int db = 0; db < DB; ++db) scale_in_place(o[hh][db], alpha);
                }
            }
            Frag8 pf[HW];
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) {
                m[hh] = mnew[hh];
                // exp2 of a masked score (-inf) is 0; the offset is kept finite so
                // that a row with nothing visible yet cannot form -inf + inf
                const float neg_m = m[hh] == -INFINITY ? 0.f : -m[hh];
                float p[2][4];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        // raw v_exp_f32: results below 2^-126 flush to zero, which is
                        // immaterial next to the row's maximum term (>= 2^-8)
                        p[kb][r] = __builtin_amdgcn_exp2f(fmaf(sc[hh][kb][r], scale_log2, neg_m));
                }
                pf[hh].w[0] = cvt_pk_bf16(p[0][0], p[0][1]);
                pf[hh].w[1] = cvt_pk_bf16(p[0][2], p[0][3]);
                pf[hh].w[2] = cvt_pk_bf16(p[1][0], p[1][1]);
                pf[hh].w[3] = cvt_pk_bf16(p[1][2], p[1][3]);
            }
            // O^T += V^T P^T; reduction slot 8g + r <-> key 4g + r, 8g + 4 + r <-> key 16 + 4g + r
            const uint16_t *va = sV + (32 * sub + 4 * g + (j >> 2)) * LDK + 4 * (j & 3);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                Frag8 vf;
                vf.h[0] = lds_read_tr16(va + 16 * db);
                vf.h[1] = lds_read_tr16(va + 16 * LDK + 16 * db);
#pragma unroll
                for (int hh = 0; hh < HW; ++hh) o[hh][db] = mfma16(vf, pf[hh], o[hh][db]);
            }
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) osum[hh] = mfma16(ones, pf[hh], osum[hh]);
        }
        if (has_next) {
            stage(buf ^ 1, sl_nxt, kx, vx);
#pragma unroll
            for (int i = 0; i < NLD; ++i) sl_nxt[i] = sl_new[i];
        }
        __syncthreads();
    }
    // finish: normalise by the row sums, store
    const int r = r0 + j;
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
        const float ls = osum[hh][0];
        if (r >= ti.rows) continue;
        const float inv = ls > 0.f ? 1.f / ls : 0.f;
        uint16_t *dst = out + (static_cast<int64_t>(ti.q0 + ti.row0 + r) * n_heads + h0 + hh) * D + 4 * g;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            uint2 w;
            w.x = cvt_pk_bf16(o[hh][db][0] * inv, o[hh][db][1] * inv);
            w.y = cvt_pk_bf16(o[hh][db][2] * inv, o[hh][db][3] * inv);
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
    const int64_t units = static_cast<int64_t>((a.num_q_tiles + kXcds - 1) / kXcds) * kXcds *
                          a.pool.n_kv_heads * C::GROUPS;
    hipLaunchKernelGGL((prefill_mfma_kernel<D, G>), dim3(static_cast<unsigned>(units)), dim3(C::THREADS),
                       0, s, static_cast<const uint16_t *>(a.q), static_cast<uint16_t *>(a.out),
                       static_cast<const uint16_t *>(a.pool.k_layer),
                       static_cast<const uint16_t *>(a.pool.v_layer), a.pool.pool_slots,
                       a.pool.n_kv_heads, a.req_to_token, a.num_reqs, a.max_ctx_len, a.req_pool_indices,
                       a.qo_indptr, a.kv_indptr, a.q_tile_to_batch, a.q_tile_to_index, a.batch,
                       a.total_q, a.n_heads, a.num_q_tiles, a.scale_log2);
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
