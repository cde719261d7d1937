// Split-K paged decode attention and its log-sum-exp merge.
//
// AstrAI docs/developer/internals.md, "KV Cache Mathematics":
// o_n = sum_j softmax(q_n k_j / sqrt(d_k)) v_j over a request's cached keys.
// docs/guides/inference.md, "KVCache System" and "Attention Backend": keys
// and values are read through req_to_token (one slot per token) at
// k/v_buffer[layer, slot, kv_head, :]; split-K writes partial outputs and
// max/log-sum partials that a second pass merges.
//
// Pass 1, one workgroup per (request b, KV head, split s) -- per (work item,
// KV head) when the step's list of (request, split) items is given, else per
// (request, split below ceil(max_len / C), KV head), where the splits past a
// request's end exit at once (on a batch of mixed lengths most of that grid;
// launching them costs the dispatcher more time than their work).  The
// split's KV positions are streamed once.  Each 16-byte slice of a KV row is read by one
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
#include <mutex>

#include "device.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace astr {
namespace {

constexpr float kLn2 = 0.693147180559945309f;

// The (KV head, split, batch entry) of this workgroup: from the work-item
// list when there is one, else from the full (entry, split, KV head) grid.
// With a list, the 8 workgroups of a group of 8 consecutive ids (dealt to
// the 8 XCDs in turn) take 8 consecutive items, and the KV head changes
// from one group to the next: every XCD then serves every KV head (giving
// each XCD one fixed KV head, as id % n_kv would, measured a 17% spread in
// per-XCD work and a 3% slower call), and the 4 KV heads of an item run on
// one XCD, sharing its L2 for the item's table reads.  False for an id past
// the list or an item outside the batch or the split axis (skipped).
__device__ __forceinline__ bool work_item(const int32_t *item_batch, const int32_t *item_index, int num_items,
                                          int batch, int n_kv, int n_splits, int &kvh, int &s, int &b) {
    if (num_items > 0) {
        const int grp = blockIdx.x >> 3;
        kvh = grp % n_kv;
        const int item = (grp / n_kv) * 8 + (blockIdx.x & 7);
        if (item >= num_items) return false;
        b = item_batch[item];
        s = item_index[item];
        return b >= 0 && b < batch && s >= 0 && s < n_splits;
    }
    kvh = blockIdx.x % n_kv;
    s = (blockIdx.x / n_kv) % n_splits;
    b = blockIdx.x / (n_kv * n_splits);
    return true;
}

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
    const int32_t *__restrict__ kv_indptr, int n_heads, int chunk, int n_splits, float scale_log2,
    const int32_t *__restrict__ item_batch, const int32_t *__restrict__ item_index, int num_items, int batch) {
    using C = DecodeCfg<T, D, G>;
    constexpr int E = C::E, LPR = C::LPR, NRG = C::NRG, U = C::U;

    int kvh, s, b;
    if (!work_item(item_batch, item_index, num_items, batch, n_kv, n_splits, kvh, s, b)) return;
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

// ---------------------------------------------------------------------------
// bf16 pass 1 on the matrix cores.
//
// One workgroup (4 waves) per (request, KV head, split); wave w takes the
// split's 32-key chunks w, w+4, ...  The chunk's K and V head rows are read
// from HBM as whole rows (D/8 consecutive lanes per 256-byte row, the pattern
// the memory system serves at streaming rate for this scattered access) with
// the non-temporal hint, and pass through a per-wave LDS tile that turns them
// into matrix-core operands.  With the G query heads of the KV head as the 16
// MFMA columns (unused columns are zero):
//   S^T[key][head] = K Q^T        A = K read back from the tile (lane: key
//                                 l%16, d = 32ks + 8(l/16)), B = Q^T kept in
//                                 registers;
//   online softmax per head       lane (g, j) holds head j's scores of keys
//                                 16kb + 4g + r;
//   O^T[d][head] += V^T P^T       B = P^T straight from the S^T accumulators
//                                 (reduction slot 8g + r <-> key 4g + r,
//                                 8g + 4 + r <-> key 16 + 4g + r), A = V^T read
//                                 from the tile with ds_read_b64_tr_b16.
// Per key and KV head this costs a 256-byte K row, a 256-byte V row, half an
// MFMA of each product and a few VALU ops for the softmax -- the VALU work of
// per-lane dot products and cross-lane reductions disappears.
//
// FUSED: the step's new token is rotated and written here (inference.md,
// "Attention Backend": the decode op takes the new k/v and writes them to the
// cache).  q arrives unrotated and every workgroup rotates its G heads at
// position L_b - 1; the wave whose chunks hold key L_b - 1 rotates k_new,
// uses it and v_new in place of that key's pool rows in its LDS tile and
// stores both into the pool (k_store / v_store alias the pool; only that wave
// loads the new token's rows, and it discards what it loaded there).
// The rotation is the one the rotary write performs, bit for bit.
// ---------------------------------------------------------------------------
template <int D, int G, bool FUSED>
__global__ __launch_bounds__(256, 3) void decode_mfma_kernel(
    const uint16_t *__restrict__ q, uint16_t *__restrict__ out, float *__restrict__ o_part,
    float *__restrict__ lse_part, const uint16_t *__restrict__ k_layer,
    const uint16_t *__restrict__ v_layer, int64_t pool_slots, int n_kv,
    const int32_t *__restrict__ req_to_token, int num_reqs, int max_ctx_len,
    const int32_t *__restrict__ req_pool_indices, const int32_t *__restrict__ kv_indptr,
    int n_heads, int chunk, int n_splits, float scale_log2, const uint16_t *__restrict__ k_new,
    const uint16_t *__restrict__ v_new, const float2 *__restrict__ tab, int max_pos, uint16_t *k_store,
    uint16_t *v_store, const int32_t *__restrict__ item_batch, const int32_t *__restrict__ item_index,
    int num_items, int batch) {
    constexpr int KS = D / 32;          // k-steps of S^T
    constexpr int DB = D / 16;          // 16-row blocks of O^T
    constexpr int CK = 32;              // keys per wave chunk
    constexpr int RB = 2 * D;           // LDS row bytes (unpadded; chunks XOR-swizzled)
    constexpr int WAVES = 4;
    static_assert(G <= 16, "query heads per KV head must fit the 16 MFMA columns");

    int kvh, s, b;
    if (!work_item(item_batch, item_index, num_items, batch, n_kv, n_splits, kvh, s, b)) return;
    const int req = req_pool_indices[b];
    const int L = request_len(kv_indptr, b, req, num_reqs, min(max_ctx_len, n_splits * chunk));
    const int start = s * chunk;
    if (start >= L && s > 0) return;
    const int end = min(start + chunk, L);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, j = lane & 15;

    // LDS: one tile per wave (the chunk's K rows, then its V rows), then the
    // cross-wave merge
    constexpr int T_BYTES = WAVES * CK * RB;
    constexpr int M_BYTES = WAVES * G * (D + 2) * 4;
    constexpr int S_BYTES = T_BYTES > M_BYTES ? T_BYTES : M_BYTES;
    constexpr int N_BYTES = FUSED ? 4 * D : 0;     // the new token's rotated k and v rows
    __shared__ __attribute__((aligned(16))) char smem[S_BYTES + N_BYTES];
    char *sT = smem + wave * CK * RB;
    uint16_t *s_new = reinterpret_cast<uint16_t *>(smem + S_BYTES);

    Frag8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks].u = j < G ? *reinterpret_cast<const uint4 *>(
                               q + (static_cast<int64_t>(b) * n_heads + kvh * G + j) * D + 32 * ks + 8 * g)
                         : make_uint4(0, 0, 0, 0);
    }
    const int npos = L - 1;                      // position of the step's new token
    const bool fuse = FUSED && npos >= 0 && npos < max_pos;
    if (fuse) {
        // rotate q: lane (g, j) holds d = 32ks + 8g .. +7 of head j, pairs 16ks + 4g ..
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            Vec<bf16_t> x;
            x.raw = qf[ks].u;
            rotate_slice(x, tab + static_cast<int64_t>(npos) * (D / 2) + 16 * ks + 4 * g);
            qf[ks].u = j < G ? x.raw : make_uint4(0, 0, 0, 0);
        }
    }
    f32x4_t o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;

    // Loads: D/8 consecutive lanes read one whole head row (256 bytes for
    // D = 128), 64/(D/8) rows per instruction, with the non-temporal hint (the
    // rows are read once).  Slots: lane l holds the slot of key c0 + (l % 32),
    // fetched one chunk ahead, and is shuffled to the lanes loading that row.
    constexpr int SL = D / 8;           // 16-byte slices per row
    constexpr int RPI = 64 / SL;        // rows per load instruction
    constexpr int NI = CK / RPI;        // load instructions per buffer per chunk
    const int rr = lane / SL, cc = lane % SL;
    // A request without keys (also one whose row index lies outside the
    // table, for which L is 0) reads row 0, which always exists.
    const int32_t *row = req_to_token + static_cast<int64_t>(L > 0 ? req : 0) * max_ctx_len;
    // Every lane reads an entry of the request's row (a key at or past `end`
    // reads entry 0 and is then marked missing): a load without a per-lane
    // branch is one the compiler can count, so the next chunk's index load
    // stays in flight while this chunk's rows are requested instead of being
    // waited for first.
    auto slot_of = [&](int c) -> int32_t {
        const int key = c + (lane & 31);
        const int32_t v = row[key < end ? key : 0];
        return key < end ? v : -1;
    };
    // the new token: lanes 0 .. D/8 - 1 of the wave whose chunks hold key
    // L - 1 rotate slice `lane` of k_new, store it and v_new into the pool and
    // stage both in LDS for that chunk's tile (only this wave loads the new
    // token's rows from the pool, and it replaces what it loaded there)
    const bool has_new = fuse && npos >= start && npos < end && ((npos - start) / CK) % WAVES == wave &&
                         rr == 0;
    if (has_new) {
        const int64_t src = (static_cast<int64_t>(b) * n_kv + kvh) * D + 8 * cc;
        Vec<bf16_t> x;
        x.raw = *reinterpret_cast<const uint4 *>(k_new + src);
        rotate_slice(x, tab + static_cast<int64_t>(npos) * (D / 2) + 4 * cc);
        const uint4 nv = *reinterpret_cast<const uint4 *>(v_new + src);
        *reinterpret_cast<uint4 *>(s_new + 8 * cc) = x.raw;
        *reinterpret_cast<uint4 *>(s_new + D + 8 * cc) = nv;
        const int64_t nslot = row[npos];
        if (nslot >= 0 && nslot < pool_slots) {
            const int64_t off = (nslot * n_kv + kvh) * D + 8 * cc;
            *reinterpret_cast<uint4 *>(k_store + off) = x.raw;
            *reinterpret_cast<uint4 *>(v_store + off) = nv;
        }
    }
    // tile byte offsets this lane writes: row i*RPI + rr, chunk cc
    int wofs[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) wofs[i] = RB * (i * RPI + rr) + 16 * (cc ^ swz<D>(i * RPI + rr));
    int32_t sl_now = slot_of(start + wave * CK);
    for (int c0 = start + wave * CK; c0 < end; c0 += WAVES * CK) {
        const int32_t sl_next = slot_of(c0 + WAVES * CK);
        uint4 kx[NI], vx[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int64_t slot = __shfl(sl_now, i * RPI + rr, 64);
            if (slot >= 0 && slot < pool_slots) {
                const int64_t off = (slot * n_kv + kvh) * D + 8 * cc;
                kx[i] = load_nt16(k_layer + off);
                vx[i] = load_nt16(v_layer + off);
            } else {
                kx[i] = make_uint4(0, 0, 0, 0);
                vx[i] = make_uint4(0, 0, 0, 0);
            }
        }
        // the chunk holding the new token: its row of the LDS tile takes the
        // rotated k_new / v_new staged above
        const bool mine = has_new && c0 <= npos && npos < c0 + CK;
        const int nofs = RB * (npos - c0) + 16 * (cc ^ swz<D>(npos - c0));
        // bit k: key c0 + k exists and has a valid slot
        const uint32_t okmask = static_cast<uint32_t>(
            __ballot(c0 + (lane & 31) < end && sl_now >= 0 && sl_now < pool_slots) & 0xffffffffull);
        // K rows -> LDS -> MFMA A-operand layout (lane: key 16kb + j, d = 32ks + 8g)
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<uint4 *>(sT + wofs[i]) = kx[i];
        if (mine) *reinterpret_cast<uint4 *>(sT + nofs) = *reinterpret_cast<const uint4 *>(s_new + 8 * cc);
        wave_lds_fence();
        Frag8 kf[2][KS];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[kb][ks].u = *reinterpret_cast<const uint4 *>(sT + RB * (16 * kb + j) + 16 * ((4 * ks + g) ^ swz<D>(j)));
        }
        wave_lds_fence();                       // K read out before V overwrites the tile
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<uint4 *>(sT + wofs[i]) = vx[i];
        if (mine) *reinterpret_cast<uint4 *>(sT + nofs) = *reinterpret_cast<const uint4 *>(s_new + D + 8 * cc);
        f32x4_t sc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sc[kb] = mfma16(kf[kb][ks], qf[ks], sc[kb]);
        }
        // online softmax of column j over keys 16kb + 4g + r
        float mx = m;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = 16 * kb + 4 * g + r;
                const float x = (okmask >> k) & 1u ? sc[kb][r] * scale_log2 : -INFINITY;
                sc[kb][r] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float alpha = exp2_sub(m, mx);
        m = mx;
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2_sub(sc[kb][r], mx);
                sc[kb][r] = p;
                ps += p;
            }
        }
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int r = 0; r < 4; ++r) o[db][r] *= alpha;
        }
        Frag8 pf;
        pf.w[0] = pack_bf16x2(sc[0][0], sc[0][1]);
        pf.w[1] = pack_bf16x2(sc[0][2], sc[0][3]);
        pf.w[2] = pack_bf16x2(sc[1][0], sc[1][1]);
        pf.w[3] = pack_bf16x2(sc[1][2], sc[1][3]);
        wave_lds_fence();                       // V tile written by all lanes of this wave
        // lane (g, j): 8 bytes at byte 8(j & 3) + 32db of row 4g + j/4 (and 16 rows on)
        const int vr = 4 * g + (j >> 2);
        const char *va = sT + RB * vr + 8 * (j & 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            Frag8 vf;
            const int vc = 16 * ((((j & 3) >> 1) + 2 * db) ^ swz<D>(vr));
            vf.h[0] = lds_read_tr16(reinterpret_cast<const uint16_t *>(va + vc));
            vf.h[1] = lds_read_tr16(reinterpret_cast<const uint16_t *>(va + 16 * RB + vc));
            o[db] = mfma16(vf, pf, o[db]);
        }
        wave_lds_fence();                       // reads done before the next chunk's writes
        sl_now = sl_next;
    }

    // row sums of each head over the 4 lane groups
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    __syncthreads();                            // V tiles are dead; reuse LDS for the merge
    float *s_m = reinterpret_cast<float *>(smem);               // [WAVES][G]
    float *s_l = s_m + WAVES * G;                               // [WAVES][G]
    float *s_o = s_l + WAVES * G;                               // [WAVES][G][D]
    if (j < G) {
        if (g == 0) {
            s_m[wave * G + j] = m;
            s_l[wave * G + j] = lsum;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int r = 0; r < 4; ++r) s_o[(wave * G + j) * D + 16 * db + 4 * g + r] = o[db][r];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 64 * WAVES) {
        const int h = idx / D, d = idx % D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) mx = fmaxf(mx, s_m[w * G + h]);
        float l = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float a = exp2_sub(s_m[w * G + h], mx);
            l += s_l[w * G + h] * a;
            acc += s_o[(w * G + h) * D + d] * a;
        }
        const float res = l > 0.f ? acc / l : 0.f;
        const int hq = kvh * G + h;
        if (n_splits == 1) {
            out[(static_cast<int64_t>(b) * n_heads + hq) * D + d] = static_cast<uint16_t>(f32_to_bf16_bits(res));
        } else {
            // The partial rows (whole 128-byte lines) go out with streaming
            // (non-temporal) stores, written back during the pass rather than
            // left dirty in L2; the 4-byte log-sum-exp entries, which share
            // lines with other splits' entries, use plain stores so that L2
            // gathers them (measured on 256 requests of 1k-32k keys: 1.8% and
            // a further 1.3% faster calls; a streaming store of the 4-byte
            // entries was slower).
            const int64_t ps = (static_cast<int64_t>(b) * n_heads + hq) * n_splits + s;
            __builtin_nontemporal_store(res, o_part + ps * D + d);
            if (d == 0) lse_part[ps] = l > 0.f ? (mx + __log2f(l)) * kLn2 : -INFINITY;
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
    // lane u holds the weight of split s0 + u; 8 partial rows in flight per lane
    float acc[PER] = {};
    float wsum = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const int sl = s0 + lane;
        const float lw = sl < ns ? lse[sl] : -INFINITY;
        const float w = lw == -INFINITY ? 0.f : __expf(lw - mx);
        wsum += w;
        const int n = min(64, ns - s0);
        for (int u0 = 0; u0 < n; u0 += 8) {
            float v[8][PER], ww[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int ss = s0 + u0 + u;
                ww[u] = __shfl(w, u0 + u, 64);
#pragma unroll
                for (int jj = 0; jj < PER; ++jj)
                    v[u][jj] = ss < ns ? op[static_cast<int64_t>(ss) * D + lane + 64 * jj] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
#pragma unroll
                for (int jj = 0; jj < PER; ++jj) acc[jj] = fmaf(ww[u], v[u][jj], acc[jj]);
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wsum += __shfl_xor(wsum, o, 64);
    T *dst = out + static_cast<int64_t>(bh) * D;
#pragma unroll
    for (int jj = 0; jj < PER; ++jj) store_scalar<T>(dst + lane + 64 * jj, wsum > 0.f ? acc[jj] / wsum : 0.f);
}

template <typename T, int D, int G>
hipError_t launch_decode_typed(const DecodeArgs &a, hipStream_t s) {
    const int n_kv = a.pool.n_kv_heads;
    const int64_t blocks = a.num_items > 0 ? static_cast<int64_t>((a.num_items + 7) / 8) * 8 * n_kv
                                           : static_cast<int64_t>(a.batch) * a.n_splits * n_kv;
    if constexpr (sizeof(T) == 2) {
        auto kern = a.k_new ? decode_mfma_kernel<D, G, true> : decode_mfma_kernel<D, G, false>;
        hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                           static_cast<const uint16_t *>(a.q), static_cast<uint16_t *>(a.out), a.o_part,
                           a.lse_part, static_cast<const uint16_t *>(a.pool.k_layer),
                           static_cast<const uint16_t *>(a.pool.v_layer), a.pool.pool_slots, n_kv,
                           a.req_to_token, a.num_reqs, a.max_ctx_len, a.req_pool_indices, a.kv_indptr,
                           a.n_heads, a.split_chunk, a.n_splits, a.scale_log2,
                           static_cast<const uint16_t *>(a.k_new), static_cast<const uint16_t *>(a.v_new),
                           reinterpret_cast<const float2 *>(a.freqs), a.max_pos,
                           static_cast<uint16_t *>(a.pool.k_layer), static_cast<uint16_t *>(a.pool.v_layer),
                           a.item_batch, a.item_index, a.num_items, a.batch);
    } else {
        hipLaunchKernelGGL((decode_split_kernel<T, D, G>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                           s, static_cast<const T *>(a.q), static_cast<T *>(a.out), a.o_part, a.lse_part,
                           static_cast<const T *>(a.pool.k_layer), static_cast<const T *>(a.pool.v_layer),
                           a.pool.pool_slots, n_kv, a.req_to_token, a.num_reqs, a.max_ctx_len,
                           a.req_pool_indices, a.kv_indptr, a.n_heads, a.split_chunk, a.n_splits,
                           a.scale_log2, a.item_batch, a.item_index, a.num_items, a.batch);
    }
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

// Split-K scratch for callers that cannot allocate: a file-scope device
// array, one copy per GPU (the runtime places it when it loads this code
// object on a device; it stays until the process ends).  Host code must not
// pass `scratch` itself to a kernel -- on the host that name is a stand-in,
// not a device address -- but the address hipGetSymbolAddress returns for
// the current device, looked up once per device and kept.
static __device__ __align__(256) float scratch[kStaticDecodeScratchBytes / sizeof(float)];

hipError_t static_decode_scratch(float **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float *by_device[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!by_device[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        by_device[dev] = static_cast<float *>(p);
    }
    *ptr = by_device[dev];
    return hipSuccess;
}

}  // namespace astr
