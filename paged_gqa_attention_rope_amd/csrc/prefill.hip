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
// Three kernels:
//  * prefill_rs (bf16, head_dim 128, a multiple of 4 query heads per KV head;
//    the one that follows a prefill work plan): 8 waves per (query tile or
//    plan unit, KV head, 4 query heads), split into score waves and output
//    waves (see the kernel).
//  * prefill_mfma (bf16, the other head counts and head_dim 64): one
//    workgroup per (query tile, KV head, pair of query heads); its 4 waves
//    hold 16 rows x 2 heads each.  Keys stream through a
//    4-deep LDS ring in steps of 32, filled by asynchronous global->LDS copies
//    issued 3 steps ahead (slot indices 5 steps ahead), so no register
//    staging and no wait for memory in the loop.  QK^T and PV run on the
//    gfx950 bf16 matrix cores (v_mfma_f32_16x16x32_bf16); the product is
//    formed transposed, S^T = K Q^T, so that a lane's accumulator registers
//    hold one query row's scores for 8 keys -- exactly the B-operand slice
//    the PV product O^T = V^T P^T needs.  P never leaves registers; V^T
//    comes from the LDS transposing read.  Online softmax in the log2 domain
//    with a lazily raised running max, fp32 accumulators, P rounded to bf16.
//  * prefill_generic (float32):
//    one workgroup per (query tile, query head), 4 lanes per query row,
//    K/V tiles of 32 keys staged in LDS as float32, online softmax per key.
#include "device.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

#include <type_traits>

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
    ti.rows = min(q_tile, ti.e - ti.row0);
    // the tile's rows must lie in [0, total_q)
    if (ti.q0 < 0 || static_cast<int64_t>(ti.q0) + ti.row0 + ti.rows > total_q) return false;
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
template <int N>
using int_c = std::integral_constant<int, N>;

template <int D, int G>
struct MfmaCfg {
    static constexpr int TQ = 64;                    // query rows per tile
    static constexpr int HW = G == 1 ? 1 : 2;        // query heads per wave
    static constexpr int GROUPS = G / HW;            // head groups per KV head
    static constexpr int WAVES = 4;                  // 4 row blocks of 16
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TS = 32;                    // keys per pipeline step
    static constexpr int NB = 4;                     // LDS ring depth, in steps
    static constexpr int AHEAD = NB - 1;             // a step's rows are requested this many steps early
    static constexpr int KS = D / 32;                // k-steps of the QK^T product
    static constexpr int DB = D / 16;                // 16-wide d blocks of the output
    static constexpr int SL = D / 8;                 // 16-byte chunks per K/V row
    static constexpr int RB = 2 * D;                 // bytes per K/V row
    static constexpr int MAT = TS * RB;              // bytes of one step's K (or V) rows
    static constexpr int RPI = 1024 / RB;            // rows one wave-wide 16-byte copy fills
    static constexpr int IPW = TS / (RPI * WAVES);   // such copies per wave, step and matrix
    static_assert(G % HW == 0 && IPW >= 1 && TS % (RPI * WAVES) == 0, "tiling");
};

// s_waitcnt immediate: at most n vector-memory operations outstanding, the
// other counters unconstrained (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most N of this wave's asynchronous copies (and other vector
// memory operations) are outstanding; also a compiler barrier for memory
// accesses, so no LDS read of copied data moves above it.
template <int N>
__device__ __forceinline__ void wait_copies() {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
    asm volatile("" ::: "memory");
}

// Workgroup barrier that orders LDS traffic without waiting for outstanding
// global->LDS copies (a full __syncthreads fence would wait for all of them):
// this wave's LDS reads and writes are complete, then all waves meet.  The
// copies a step needs are waited for explicitly, by count, before it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8_t *)p));
}

// Asynchronous global->LDS copies: lane l's 16 (4) bytes land at LDS address
// lds + 16*l (4*l); lds must be wave-uniform.  Written as inline assembly so
// that the compiler does not track them: it would otherwise make the LDS
// reads of other ring slots wait for them.  Their completion is waited for
// explicitly, by count, before the barrier that publishes the data.  (One
// wait state separates the M0 write from the copy that reads it.)
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// 16 bytes at byte `off` of record `idx` of the structured buffer `rsrc`; a
// record index at or past the buffer's record count reads zeros (the
// hardware range check).
__device__ __forceinline__ void copy_record16_to_lds(i32x4_t rsrc, uint32_t idx, uint32_t off, uint32_t lds) {
    const u32x2_t a = {idx, off};
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 idxen offen lds" ::"v"(a),
                 "s"(rsrc), "s"(lds)
                 : "memory", "m0");
}
// 4 bytes at byte voff of the raw buffer `rsrc`; bytes at or past its size
// read zeros and touch no memory.  The whole offset goes in the VGPR offset:
// the hardware range check of a raw buffer covers the VGPR and instruction
// offsets only, not the SGPR offset.
__device__ __forceinline__ void copy_raw4_to_lds(i32x4_t rsrc, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
                 "s"(lds)
                 : "memory", "m0");
}

// Buffer resource (gfx9 layout) over `records` records of `stride` bytes.
__device__ __forceinline__ i32x4_t buffer_rsrc(const void *base, uint32_t stride, uint32_t records) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r.x = static_cast<int>(static_cast<uint32_t>(a));
    r.y = static_cast<int>((static_cast<uint32_t>(a >> 32) & 0xffffu) | (stride << 16));
    r.z = static_cast<int>(records);
    r.w = 0x00020000;                                // 32-bit data format: raw loads enabled
    return r;
}

// One workgroup per (query tile, KV head, head group of HW query heads).
// Wave w owns query rows 16w .. 16w+15 of the tile for the HW heads, so every K
// and V operand read from LDS feeds HW matrix-core products; it keeps the
// Q^T operands and O^T accumulators in registers.
//
// Keys are processed in steps of 32 through a ring of 4 LDS slots (K and V
// rows of one step each), filled by asynchronous global->LDS copies issued 3
// steps ahead, whose slot indices are fetched one step before that.  Step s:
//   barrier (the copies of step s+1 have landed, everyone is done with s-1);
//   S^T(s+1) = K(s+1) Q^T on the matrix cores while P(s) = exp2(S(s) - m)
//   is formed on the vector ALUs; O^T += V(s)^T P(s)^T while the row maxima
//   of S(s+1) are formed; mask S(s+1) where it crosses the causal diagonal or
//   has a missing slot; raise the running max only when a row's max grew by
//   more than 8 (exact: the same stale max enters numerator and denominator,
//   and probabilities stay below 2^8); request step s+3's rows.
// Row sums come from the matrix cores (P^T against a ones operand).
template <int D, int G, bool WIDE>
__global__ __launch_bounds__((MfmaCfg<D, G>::THREADS), 2) void prefill_mfma_kernel(
    const uint16_t *__restrict__ q, uint16_t *__restrict__ out, const uint16_t *__restrict__ k_layer,
    const uint16_t *__restrict__ v_layer, int64_t pool_slots, int n_kv,
    const int32_t *__restrict__ req_to_token, int num_reqs, int max_ctx_len,
    const int32_t *__restrict__ req_pool_indices, const int32_t *__restrict__ qo_indptr,
    const int32_t *__restrict__ kv_indptr, const int32_t *__restrict__ q_tile_to_batch,
    const int32_t *__restrict__ q_tile_to_index, int batch, int total_q, int n_heads,
    int num_q_tiles, float scale_log2) {
    using C = MfmaCfg<D, G>;
    constexpr int TQ = C::TQ, HW = C::HW, KS = C::KS, DB = C::DB, SL = C::SL, RB = C::RB;
    constexpr int MAT = C::MAT, TS = C::TS, NB = C::NB, AHEAD = C::AHEAD, RPI = C::RPI, IPW = C::IPW;
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
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, j = lane & 15;
    const int r0 = 16 * wave;                        // first tile row of this wave
    const int h0 = kvh * G + grp * HW;               // first query head of this wave
    const int qpos0 = ti.p + ti.row0 + r0;           // position of the wave's first row
    const int qpos = qpos0 + j;                      // position of this lane's row
    const int nsteps = (ti.kv_end + TS - 1) / TS;

    // the ring: slot i holds one step's K rows, then its V rows
    __shared__ __attribute__((aligned(1024))) uint8_t ring0[2 * MAT], ring1[2 * MAT], ring2[2 * MAT],
        ring3[2 * MAT];
    __shared__ uint32_t badf[NB];                    // per step: keys whose slot lies outside the pool
    auto ring = [&](auto rc) -> uint8_t * {
        constexpr int R = decltype(rc)::value;
        if constexpr (R == 0) return ring0;
        else if constexpr (R == 1) return ring1;
        else if constexpr (R == 2) return ring2;
        else return ring3;
    };

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
    // running row max m (log2 domain, scaled), -m as the exponent offset (0
    // while nothing is visible, so that -inf + inf never forms), and the raw
    // score above which a lane's scores call for a larger m
    float m[HW], neg_m[HW], thr[HW];
    const float inv_scale = 1.f / scale_log2;
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
        m[hh] = -INFINITY;
        neg_m[hh] = 0.f;
        thr[hh] = -INFINITY;
        osum[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < DB; ++db) o[hh][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    Frag8 ones;                                      // bf16 1.0 in every reduction slot
    ones.u = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);

    // LDS read offsets within a slot.  K operand (key block kb, k-step ks) of
    // lane (g, j): row 16kb + j, chunk 4ks + g; V^T operand (d block db) via the
    // transposing read: lane (g, j) points at row 4g + j/4 (+16 for the second
    // half), elements 16db + 4(j%4) .. +3.  The swizzle only permutes chunks
    // inside a row and repeats every 16 rows, so both become a per-lane base
    // XOR a per-block constant.
    uint32_t kofs[KS], vofs[DB];
    {
        const uint32_t kb0 = RB * j + 16 * (g ^ swz<D>(j));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kofs[ks] = kb0 ^ (64 * ks);
        const int vr = 4 * g + (j >> 2);
        const uint32_t vb0 = RB * vr + 8 * (j & 1) + 16 * (((j & 3) >> 1) ^ swz<D>(vr));
#pragma unroll
        for (int db = 0; db < DB; ++db) vofs[db] = vb0 ^ (32 * db);
    }

    // Copies: copy c (0..IPW-1) of this wave fills step rows RPI*(IPW*wave+c) ..
    // +RPI-1; lane l writes chunk position l % SL of row RPI*(IPW*wave+c) + l/SL,
    // so it reads that row's chunk (l % SL) ^ swz(row).
    const int crow = RPI * IPW * wave + lane / SL;
    uint32_t ccol[IPW];
#pragma unroll
    for (int c = 0; c < IPW; ++c) ccol[c] = (WIDE ? 0 : kvh * RB) + 16 * ((lane % SL) ^ swz<D>(crow + RPI * c));
    const int32_t *trow = req_to_token + static_cast<int64_t>(ti.req) * max_ctx_len;
    // The pool as a structured buffer: records are slots (stride n_kv*RB, at
    // most 16383 bytes), or, for wider slots, (slot, KV head) rows of RB bytes.
    const uint32_t slot_lim = static_cast<uint32_t>(min(pool_slots, static_cast<int64_t>(INT32_MAX)));
    const uint32_t stride = WIDE ? RB : static_cast<uint32_t>(n_kv) * RB;
    const uint32_t records = WIDE ? static_cast<uint32_t>(min(static_cast<int64_t>(slot_lim) * n_kv,
                                                              static_cast<int64_t>(UINT32_MAX)))
                                  : slot_lim;
    const i32x4_t krs = buffer_rsrc(k_layer, stride, records);
    const i32x4_t vrs = buffer_rsrc(v_layer, stride, records);

    // Slot indices travel the same way as the rows: wave w's 8 rows of step t
    // (rows 8w .. 8w+7) have their req_to_token entries copied into that
    // wave's part of a small LDS ring two steps before the rows are requested.
    // (Keys past the tile's last visible key take the last one's entry: valid
    // rows, masked by causality.)  All vector-memory operations of the loop are
    // then asynchronous LDS copies, which retire in order, so the explicit
    // wait counts below are exact.
    static_assert(RPI * IPW == 8, "8 rows per wave and step");
    __shared__ int32_t sidx0[C::WAVES][8], sidx1[C::WAVES][8], sidx2[C::WAVES][8], sidx3[C::WAVES][8];
    auto sidx = [&](auto rc) -> int32_t * {
        constexpr int R = decltype(rc)::value;
        if constexpr (R == 0) return sidx0[wave];
        else if constexpr (R == 1) return sidx1[wave];
        else if constexpr (R == 2) return sidx2[wave];
        else return sidx3[wave];
    };
    // the request's table row up to its last visible key; entries past it
    // (steps fetched ahead of the last one) read 0 without touching memory
    const i32x4_t trs = buffer_rsrc(trow, 0, 4u * static_cast<uint32_t>(ti.kv_end));
    const uint32_t idx_voff = 4u * (8 * wave + lane);
    auto fetch_idx = [&](auto rc, int t) {
        if (lane < 8) copy_raw4_to_lds(trs, idx_voff + 4u * TS * t, lds_addr(sidx(rc)));
    };
    // A key whose slot lies outside the pool, and every key of a step
    // t >= nsteps (whose rows are never used; copying zeros keeps the number
    // of copies per step, and so the explicit wait counts, the same on every
    // path), gets an out-of-range record index: its K and V rows read zeros.
    auto issue = [&](auto rc, int t) {
        constexpr int R = decltype(rc)::value;
        uint8_t *dst = ring(rc);
        const int32_t *ix = sidx(rc);
        const int lim = ti.kv_end - TS * t;         // keys of step t at or past this row are not visible
        int32_t sls[IPW];                            // all indices first: one LDS round trip
#pragma unroll
        for (int c = 0; c < IPW; ++c) sls[c] = ix[lane / SL + RPI * c];
        bool ok[IPW], bad = false;
#pragma unroll
        for (int c = 0; c < IPW; ++c) {
            ok[c] = static_cast<uint32_t>(sls[c]) < slot_lim;
            bad = bad || !ok[c];
        }
        // record index: the slot (past the pool: zeros by the range check), or
        // (slot, KV head) for wide slots; out of range past the visible keys
        uint32_t rec[IPW];
#pragma unroll
        for (int c = 0; c < IPW; ++c) {
            if constexpr (WIDE) rec[c] = ok[c] ? static_cast<uint32_t>(sls[c]) * n_kv + kvh : 0xffffffffu;
            else rec[c] = static_cast<uint32_t>(sls[c]);
        }
        if (lim < TS) {                              // the request's last step, or past it
#pragma unroll
            for (int c = 0; c < IPW; ++c)
                if (crow + RPI * c >= lim) rec[c] = 0xffffffffu;
        }
#pragma unroll
        for (int c = 0; c < IPW; ++c) {
            const uint32_t dk = lds_addr(dst) + RB * RPI * (IPW * wave + c);
            copy_record16_to_lds(krs, rec[c], ccol[c], dk);
            copy_record16_to_lds(vrs, rec[c], ccol[c], dk + MAT);
        }
        // this wave's 8 rows (8w .. 8w+7) of the step's missing-slot mask
        uint32_t byte = 0;
        if (__builtin_expect(__any(bad), 0)) {
#pragma unroll
            for (int c = 0; c < IPW; ++c) {
                const uint64_t b = __ballot(!ok[c]);
#pragma unroll
                for (int r = 0; r < RPI; ++r)
                    if ((b >> (r * SL)) & 1u) byte |= 1u << (RPI * c + r);
            }
        }
        if (lane == 0) reinterpret_cast<uint8_t *>(&badf[R])[wave] = static_cast<uint8_t>(byte);
    };

    // K operands of a step (key block kb, k-step ks)
    auto load_k = [&](auto rc, Frag8 (&kf)[KS][2]) {
        const uint8_t *base = ring(rc);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                kf[ks][kb].u = *reinterpret_cast<const uint4 *>(base + 16 * RB * kb + kofs[ks]);
        }
    };
    // V^T operands of a step (d block db); reduction slot 8g + r <-> key
    // 4g + r, 8g + 4 + r <-> key 16 + 4g + r
    auto load_v = [&](auto rc, Frag8 (&vf)[DB]) {
        const uint8_t *vbase = ring(rc) + MAT;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            vf[db].h[0] = lds_read_tr16(reinterpret_cast<const uint16_t *>(vbase + vofs[db]));
            vf[db].h[1] = lds_read_tr16(reinterpret_cast<const uint16_t *>(vbase + 16 * RB + vofs[db]));
        }
    };
    // S^T = K Q^T
    auto qk = [&](const Frag8 (&kf)[KS][2], f32x4_t (&sc)[HW][2]) {
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
            sc[hh][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            sc[hh][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int hh = 0; hh < HW; ++hh) sc[hh][kb] = mfma16(kf[ks][kb], qf[hh][ks], sc[hh][kb]);
            }
        }
    };
    // P = exp2(S * scale - m) rounded to bf16, as the B operand of the PV product
    auto probs = [&](const f32x4_t (&sc)[HW][2], Frag8 (&pf)[HW]) {
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
            // exp2 of a masked score (-inf) is 0
            float p[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    // raw v_exp_f32: results below 2^-126 flush to zero, which is
                    // immaterial next to the row's maximum term (>= 2^-8)
                    p[kb][r] = __builtin_amdgcn_exp2f(fmaf(sc[hh][kb][r], scale_log2, neg_m[hh]));
            }
            pf[hh].w[0] = cvt_pk_bf16(p[0][0], p[0][1]);
            pf[hh].w[1] = cvt_pk_bf16(p[0][2], p[0][3]);
            pf[hh].w[2] = cvt_pk_bf16(p[1][0], p[1][1]);
            pf[hh].w[3] = cvt_pk_bf16(p[1][2], p[1][3]);
        }
    };
    // O^T += V^T P^T, and the row sums of P
    auto pv = [&](const Frag8 (&vf)[DB], const Frag8 (&pf)[HW]) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) o[hh][db] = mfma16(vf[db], pf[hh], o[hh][db]);
        }
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) osum[hh] = mfma16(ones, pf[hh], osum[hh]);
    };
    // raw maxima of this lane's 8 scores per head
    auto local_max = [&](const f32x4_t (&sc)[HW][2], float (&lm)[HW]) {
#pragma unroll
        for (int hh = 0; hh < HW; ++hh)
            lm[hh] = fmaxf(fmaxf(fmaxf(sc[hh][0][0], sc[hh][0][1]), fmaxf(sc[hh][0][2], sc[hh][0][3])),
                           fmaxf(fmaxf(sc[hh][1][0], sc[hh][1][1]), fmaxf(sc[hh][1][2], sc[hh][1][3])));
    };
    // keys of this lane: kb0 + 16kb + 4g + r; row: qpos
    auto apply_mask = [&](f32x4_t (&sc)[HW][2], int kb0, uint32_t okw) {
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
    };
    // Raise the running max of the rows where a score exceeds it by more than
    // kLazy.  Each lane tests its own scores against thr; only when some lane
    // of the wave fires (rarely, after the first steps) are the row maxima
    // formed across the four lanes of each row -- so the new max is the same
    // on all of them -- and the accumulators rescaled.
    auto update_max = [&](const float (&lm)[HW]) {
        bool fire = false;
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) fire = fire || lm[hh] > thr[hh];
        if (__builtin_expect(__any(fire), 0)) {
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) {
                const float mx = max_over_groups(lm[hh]) * scale_log2;   // scale > 0 keeps the order
                const float mnew = mx > m[hh] + kLazy ? mx : m[hh];
                const float alpha = exp2_sub(m[hh], mnew);                // 1 where m is unchanged
                scale_in_place(osum[hh], alpha);
#pragma unroll
                for (int db = 0; db < DB; ++db) scale_in_place(o[hh][db], alpha);
                m[hh] = mnew;
                neg_m[hh] = mnew == -INFINITY ? 0.f : -mnew;
                thr[hh] = (mnew + kLazy) * inv_scale;
            }
        }
    };
    // mask bits of the keys of a step whose slot lies in the pool
    auto ok_mask = [&](auto rc) -> uint32_t {
        constexpr int R = decltype(rc)::value;
        return ~static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(badf[R])));
    };
    // mask where step t crosses the causal diagonal or has a missing slot
    auto mask_step = [&](auto rc, f32x4_t (&sc)[HW][2], int t, float (&lm)[HW]) {
        const uint32_t okw = ok_mask(rc);
        const int kb0 = TS * t;
        if (kb0 + TS - 1 > qpos0 || okw != 0xffffffffu) {
            apply_mask(sc, kb0, okw);
            local_max(sc, lm);
        }
    };

    // prologue: the steady-state issue sequence of steps -3 .. -1 (indices of
    // step t+5, then the rows of step t+3; the indices a copy needs must have
    // landed before they are read,
    f32x4_t sA[HW][2], sB[HW][2];                   // scores, by step parity
    // and each wait names the copies issued after the one it needs)
    fetch_idx(int_c<0>{}, 0);
    fetch_idx(int_c<1>{}, 1);
    fetch_idx(int_c<2>{}, 2);
    wait_copies<2>();                                  // indices of step 0
    issue(int_c<0>{}, 0);
    fetch_idx(int_c<3>{}, 3);
    wait_copies<2 * IPW + 2>();                        // indices of step 1
    issue(int_c<1>{}, 1);
    fetch_idx(int_c<0>{}, 4);
    wait_copies<4 * IPW + 2>();                        // indices of step 2
    issue(int_c<2>{}, 2);
    wait_copies<4 * IPW + 2>();                        // rows of step 0
    lds_barrier();
    {
        Frag8 kf[KS][2];
        load_k(int_c<0>{}, kf);
        qk(kf, sA);
    }
    {
        float lm[HW];
        local_max(sA, lm);
        mask_step(int_c<0>{}, sA, 0, lm);
        update_max(lm);
    }

    // one pipeline step; true after the last one
    auto step = [&](auto rc, int s, f32x4_t (&sc)[HW][2], f32x4_t (&sn)[HW][2]) -> bool {
        constexpr int R = decltype(rc)::value;
        constexpr int R1 = (R + 1) % NB, R3 = (R + AHEAD) % NB;
        // the rows of step s+1 have landed (those of s+2 may still be in flight:
        // 2*IPW+1 copies were issued after them)
        wait_copies<2 * IPW + 1>();
        lds_barrier();
        const bool more = s + 1 < nsteps;
        // all LDS operands of the step first (K of step s+1, V of step s), then
        // S of step s+1 on the matrix cores interleaved with this step's
        // probabilities on the vector ALUs, then O += V P interleaved with the
        // lane maxima of S(s+1) (S of the step after the last is unused)
        Frag8 kf[KS][2], vf[DB], pf[HW];
        load_k(int_c<R1>{}, kf);
        load_v(rc, vf);
        qk(kf, sn);
        probs(sc, pf);
        pv(vf, pf);
        float lm[HW];
        local_max(sn, lm);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS + 2 * DB, 0);     // LDS reads
#pragma unroll
        for (int i = 0; i < 2 * KS * HW; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);               // three VALU
        }
#pragma unroll
        for (int i = 0; i < DB * HW + HW; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
        }
        if (more) {
            mask_step(int_c<R1>{}, sn, s + 1, lm);
            update_max(lm);
        }
        // indices of step s+5, then the rows of step s+3 (their indices, copied
        // two steps ago, landed before this step's barrier)
        fetch_idx(int_c<(R + 1) % NB>{}, s + AHEAD + 2);
        issue(int_c<R3>{}, s + AHEAD);
        return !more;
    };
    for (int s = 0;; s += NB) {
        if (step(int_c<0>{}, s, sA, sB)) break;
        if (step(int_c<1>{}, s + 1, sB, sA)) break;
        if (step(int_c<2>{}, s + 2, sA, sB)) break;
        if (step(int_c<3>{}, s + 3, sB, sA)) break;
    }
    wait_copies<0>();                                // no copy outlives the workgroup

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

// Keep a value's computation before this point: an empty asm that reads and
// rewrites the registers (volatile asm statements keep their order, and the
// phase barriers are volatile asm).
__device__ __forceinline__ void pin(Frag8 &x) { asm volatile("" : "+v"(x.v)); }
__device__ __forceinline__ void pin(f32x4_t &x) { asm volatile("" : "+v"(x)); }
template <typename T, int N>
__device__ __forceinline__ void pin(T (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) pin(x[i]);
}

// ---------------------------------------------------------------------------
// role-split kernel: D = 128, a multiple of 4 query heads per KV head
// ---------------------------------------------------------------------------
// One workgroup of 8 waves per (query tile or plan unit, KV head, 4 query
// heads).  Waves 0-3 are score waves: wave w holds rows 16w .. 16w+15 of the
// tile for all 4 heads, forms S(t) = K(t) Q^T on the matrix cores, masks it,
// keeps the running max and writes P(t) = exp2(S(t) - m) (bf16, in the
// matrix-core operand layout) to an LDS ring.  Waves 4-7 are output waves:
// wave 4+w holds the O^T accumulators of the same rows and heads and, one
// step later, reads P(t) and V(t) and adds O^T += V^T P^T (and the row sums
// against a ones operand).  Waves w and w+4 share a SIMD, so one runs mostly
// products and the other the vector work of the softmax; the score waves
// raise their priority while they issue their products, so that those go
// first and the output waves' products fill the matrix core while the score
// waves form P.  Each K and V operand is read from LDS once per wave that
// needs it (four times per step each); a score wave reads the K operands of
// step t+1 during step t, after issuing the products of S(t), so that its
// products start at the barrier instead of behind the burst of LDS reads
// that follows it.  One barrier per step: in iteration t
// the score waves form P(t) while the output waves consume P(t-1).  A raise
// of the running max travels with P (a flag, set only on a raise and cleared
// by the output wave that reads it, and the per-row factors), and the output
// waves rescale before adding.
// Keys arrive through a ring of 6 LDS slots by asynchronous copies issued 4
// steps ahead by the 4 output waves (slot indices 6 steps ahead); every wait
// is an explicit count.  The score waves, which set the pace of a step, issue
// no copies, and their common path holds only the products, the max test,
// exp2 and the packing: each vector instruction taken off it measured worth
// ~15-20 cycles of the step.  Steps are numbered from the unit's first step
// t0; ring slot and P slot follow t - t0.
// Q is multiplied by scale*log2(e) and rounded to bf16 once, when it is
// loaded, and every score accumulator starts at -m (the running max), so the
// products deliver the exponent itself and P needs only the exp2 and the
// bf16 packing (the extra rounding of Q adds a relative error of at most 2^-9
// per element of q; on the radix-prefix batch the relative L2 error against
// the float64 definition goes from 2.4e-3 to 2.9e-3).  The keys of a step
// whose slot lies outside the pool are found by one ballot over its 32 slot
// indices, and the raise test of the running max is one ballot: the max of
// the lane's 32 scores (4 heads) against the smallest of the heads'
// thresholds (the heads share the rows and the mask, so their thresholds
// move together; a raise recomputes each head's max).
// Measured against an earlier design of this kernel, where two groups of 4
// waves alternated product and vector phases with a barrier per phase: 3-6%
// faster on 16 requests with radix prefixes, ~2% on 64 requests of 2048
// cached + 64 new tokens, same error.
struct RsCfg {
    static constexpr int D = 128, TQ = 64, HW = 4, WAVES = 8, THREADS = 64 * WAVES;
    static constexpr int TS = 32, NB = 6, NI = 8;     // keys per step, ring slots, index slots
    static constexpr int KS = D / 32, DB = D / 16, SL = D / 8, RB = 2 * D, MAT = TS * RB;
    static constexpr int SLOT = 2 * MAT;               // one step's K rows, then its V rows
    static constexpr int RPI = 1024 / RB;              // rows one wave-wide 16-byte copy fills
    static constexpr int PSLOT = 4 * HW * 64 * 16;     // one step's P of the 4 score waves
    static_assert(2 * RPI * (WAVES / 2) == TS, "two K and two V copies per output wave and step");
};

template <int G, bool WIDE>
__global__ __launch_bounds__(RsCfg::THREADS, 1) void prefill_rs_kernel(
    const uint16_t *__restrict__ q, uint16_t *__restrict__ out, const uint16_t *__restrict__ k_layer,
    const uint16_t *__restrict__ v_layer, int64_t pool_slots, int n_kv,
    const int32_t *__restrict__ req_to_token, int num_reqs, int max_ctx_len,
    const int32_t *__restrict__ req_pool_indices, const int32_t *__restrict__ qo_indptr,
    const int32_t *__restrict__ kv_indptr, const int32_t *__restrict__ q_tile_to_batch,
    const int32_t *__restrict__ q_tile_to_index, int batch, int total_q, int n_heads,
    int num_q_tiles, float scale_log2, const int32_t *__restrict__ units, int num_units, int num_pairs,
    int32_t *__restrict__ part_cnt, float *__restrict__ part) {
    using C = RsCfg;
    constexpr int D = C::D, TQ = C::TQ, HW = C::HW, KS = C::KS, DB = C::DB, SL = C::SL, RB = C::RB;
    constexpr int MAT = C::MAT, SLOT = C::SLOT, TS = C::TS, NB = C::NB, NI = C::NI, RPI = C::RPI;
    constexpr int WAVES = C::WAVES, PSLOT = C::PSLOT;
    constexpr int GROUPS = G / 4;                      // workgroups per KV head
    constexpr float kLazy = 8.f;
    static_assert(G % 4 == 0, "4 query heads per workgroup");

    // units (tiles, or the key halves of a plan's split tiles) dealt to the
    // 8 XCDs in list order, heaviest first, as in prefill_mfma_kernel
    const int units_per_tile = n_kv * GROUPS;
    const int xcd = blockIdx.x % kXcds, k_in = blockIdx.x / kXcds;
    const int unit = kXcds * (k_in / units_per_tile) + xcd;
    const int u = k_in % units_per_tile;
    const int kvh = u / GROUPS;
    const int hg = u % GROUPS;
    int step_lo = 0, step_hi = INT_MAX, pw = -1;
    TileInfo ti;
    if (num_units > 0) {
        // the plan states the unit's rows and keys: one load, where the tile
        // maps would take two dependent ones
        if (unit >= num_units) return;
        const int4 d0 = reinterpret_cast<const int4 *>(units)[2 * unit];
        const int4 d1 = reinterpret_cast<const int4 *>(units)[2 * unit + 1];
        step_lo = d0.y;
        step_hi = d0.z;
        pw = d0.w < 0 ? -1 : d0.w;
        ti.req = d1.x;
        ti.q0 = d1.y;
        ti.row0 = 0;
        ti.rows = d1.z;
        ti.p = d1.w;
        if (step_lo < 0 || pw >= 2 * num_pairs || ti.rows < 1 || ti.rows > TQ || ti.req < 0 ||
            ti.req >= num_reqs || ti.q0 < 0 || ti.q0 > total_q - ti.rows || ti.p < 0 ||
            ti.p > max_ctx_len - ti.rows)
            return;                                    // not a unit of a plan for this call
        ti.kv_end = ti.p + ti.rows;
    } else {
        if (unit >= num_q_tiles ||
            !tile_info(unit, q_tile_to_batch, q_tile_to_index, qo_indptr, kv_indptr, req_pool_indices,
                       batch, num_reqs, max_ctx_len, total_q, TQ, ti))
            return;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int outw = __builtin_amdgcn_readfirstlane(wave >= 4 ? 1 : 0);   // output wave
    const int g = lane >> 4, j = lane & 15;
    const int rb = wave & 3;                           // row block of this wave
    const int r0 = 16 * rb;
    const int h0 = kvh * G + 4 * hg;                   // first of the 4 query heads
    const int qpos0 = ti.p + ti.row0 + r0;
    const int qpos = qpos0 + j;
    // this unit's key steps [t0, t1), and the keys its copies may fetch
    const int t0 = step_lo;
    const int t1 = min(step_hi, (ti.kv_end + TS - 1) / TS);
    const int kv_lim = min(ti.kv_end, TS * t1);
    // This wave pair's own steps [t0, t1w): every key of a later step lies
    // past the last of its rows (causal mask), and rows past the tile's end
    // have no steps, so those products and exponentials would only add zeros.
    // The pair still takes part in every copy and barrier up to t1.
    const int t1w = r0 < ti.rows ? min(t1, (ti.p + ti.row0 + min(r0 + 15, ti.rows - 1)) / TS + 1) : t0;

    __shared__ __attribute__((aligned(1024))) uint8_t ring[NB * SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t pring[2 * PSLOT];   // P of steps t - t0 = 0, 1 mod 2
    __shared__ float alpha_s[2][4][HW][16];            // per P slot, row block, head, row
    __shared__ uint32_t aflag[2][4];                   // a raise of the max in that step
    __shared__ int32_t sidx[NI][WAVES][RPI];           // slot indices of a step's rows
    __shared__ float m_s[4][HW][16];                   // running max handed to the output waves
    __shared__ int32_t seen;                           // a split half's completion count
    auto slot_ptr = [&](auto rc) -> uint8_t * {
        constexpr int R = decltype(rc)::value;
        return ring + R * SLOT;
    };

    // ---- copies (output waves): output wave ow fills rows 8ow .. 8ow+7 of a
    // step (two wave-wide copies of 4 rows for K and for V) and fetches the
    // slot indices of those keys ----
    const int ow = wave & 3;
    int crow[2];
    uint32_t ccol[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        crow[c] = 8 * ow + RPI * c + lane / SL;
        ccol[c] = (WIDE ? 0 : kvh * RB) + 16 * ((lane % SL) ^ swz<D>(crow[c]));
    }
    const int32_t *trow = req_to_token + static_cast<int64_t>(ti.req) * max_ctx_len;
    const uint32_t slot_lim = static_cast<uint32_t>(min(pool_slots, static_cast<int64_t>(INT32_MAX)));
    const uint32_t stride = WIDE ? RB : static_cast<uint32_t>(n_kv) * RB;
    const uint32_t records = WIDE ? static_cast<uint32_t>(min(static_cast<int64_t>(slot_lim) * n_kv,
                                                              static_cast<int64_t>(UINT32_MAX)))
                                  : slot_lim;
    const i32x4_t krs = buffer_rsrc(k_layer, stride, records);
    const i32x4_t vrs = buffer_rsrc(v_layer, stride, records);
    const i32x4_t trs = buffer_rsrc(trow, 0, 4u * static_cast<uint32_t>(ti.kv_end));
    const uint32_t idx_voff = 4u * (8 * ow + lane);
    const uint32_t sidx_base = lds_addr(sidx) + 4u * 8 * ow;
    // slot indices of step t's keys 8ow .. 8ow+7 into index slot t % NI
    auto fetch_idx = [&](int t) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(sidx_base + 4u * TS * (t & (NI - 1)));
        if (lane < 8) copy_raw4_to_lds(trs, idx_voff + 4u * TS * t, dst);
    };
    // this wave's slot indices of step t's rows (their index copies landed)
    auto slot_index = [&](int t, int32_t (&sl)[2]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) sl[c] = (&sidx[t & (NI - 1)][0][0])[crow[c]];
    };
    // rows of step t into ring slot R with slot indices sl2; t >= t1, or past
    // the visible keys: out-of-range records, which read zeros (the copy
    // count never changes)
    auto issue = [&](auto rc, int t, const int32_t (&sl2)[2]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int32_t sl = sl2[c];
            const bool ok = static_cast<uint32_t>(sl) < slot_lim;
            uint32_t rec;
            if constexpr (WIDE) rec = ok ? static_cast<uint32_t>(sl) * n_kv + kvh : 0xffffffffu;
            else rec = static_cast<uint32_t>(sl);
            if (crow[c] >= kv_lim - TS * t) rec = 0xffffffffu;
            const uint32_t dk = lds_addr(slot_ptr(rc)) + RB * (8 * ow + RPI * c);
            copy_record16_to_lds(krs, rec, ccol[c], dk);
            copy_record16_to_lds(vrs, rec, ccol[c], dk + MAT);
        }
    };
    // bit k: key k of step t has its slot in the pool (the 32 slot indices of
    // a step lie contiguously in its index slot; every wave's index copy of
    // step t landed before it issued its rows of t, several barriers ago)
    auto idx_of_step = [&](int t) -> int32_t { return (&sidx[t & (NI - 1)][0][0])[lane & 31]; };
    auto ok_bits = [&](int32_t ix) -> uint32_t {
        return static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(static_cast<uint32_t>(ix) < slot_lim));
    };
    // a step ends: this wave's LDS traffic is complete, then all waves meet;
    // no instruction moves across it
    auto phase_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // this lane's 16-byte P slice of head hh in P slot P
    auto p_addr = [&](auto pc, int hh) -> uint8_t * {
        constexpr int P = decltype(pc)::value;
        return pring + P * PSLOT + ((rb * HW + hh) * 64 + lane) * 16;
    };
    if (tid < 8) (&aflag[0][0])[tid] = 0u;          // no raise yet (the prologue's barrier publishes it)
    // prologue (output waves): indices of steps t0..t0+5, rows of steps
    // t0..t0+3, in the order that leaves exactly 10 copies after the rows of
    // step t0+2 at the end of the first iteration (as after the rows of step
    // t+2 at the end of iteration t); each index copy is waited for by the
    // count issued after it, and the rows of steps t0 and t0+1 before the
    // barrier, which the score waves meet
    auto prologue = [&]() {
        if (outw) {
            fetch_idx(t0);
            fetch_idx(t0 + 1);
            fetch_idx(t0 + 2);
            wait_copies<2>();                          // indices of step t0
            {
                int32_t sl[2];
                slot_index(t0, sl);
                issue(int_c<0>{}, t0, sl);
            }
            fetch_idx(t0 + 3);
            wait_copies<6>();
            {
                int32_t sl[2];
                slot_index(t0 + 1, sl);
                issue(int_c<1>{}, t0 + 1, sl);
            }
            fetch_idx(t0 + 4);
            wait_copies<10>();
            {
                int32_t sl[2];
                slot_index(t0 + 2, sl);
                issue(int_c<2>{}, t0 + 2, sl);
            }
            fetch_idx(t0 + 5);
            wait_copies<10>();
            {
                int32_t sl[2];
                slot_index(t0 + 3, sl);
                issue(int_c<3>{}, t0 + 3, sl);
            }
            wait_copies<10>();                         // rows of steps t0 and t0 + 1
        }
        phase_end();
    };

    // Every iteration t (t0 .. t1, one barrier each): the output waves first
    // take their slot indices of step t+4 (9 copies were issued after them);
    // after their products, the indices of step t+6 and the rows of step t+4,
    // then the wait for the rows of step t+2 (10 copies were issued after
    // them; the score waves read the K operands of step t+1 in iteration t).
    // The two roles run apart (their barriers meet: every wave of the
    // workgroup passes the same number of them in the same order).
    constexpr int64_t kPart = kPrefillPartFloats;
    constexpr int kML = 4 * HW * DB * 4 * 64;          // offset of (m, l) in a workspace part
    static_assert(kML + 4 * HW * 64 * 2 == kPart, "workspace layout");
    const int64_t ps = (static_cast<int64_t>(pw < 0 ? 0 : pw >> 1) * n_kv + kvh) * GROUPS + hg;   // part slot
    if (!outw) {
        // ================= score waves =================
        float m[HW];                                   // running row max (log2 domain)
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) m[hh] = -INFINITY;
        if (t0 < t1) {
        Frag8 qf[HW][KS];
        {
            int r = r0 + j;
            if (r >= ti.rows) r = 0;
            const uint16_t *src = q + (static_cast<int64_t>(ti.q0 + ti.row0 + r) * n_heads + h0) * D + 8 * g;
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    Frag8 raw;
                    raw.u = *reinterpret_cast<const uint4 *>(src + hh * D + 32 * ks);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = __uint_as_float(raw.w[e] << 16) * scale_log2;
                        const float hi = __uint_as_float(raw.w[e] & 0xffff0000u) * scale_log2;
                        qf[hh][ks].w[e] = cvt_pk_bf16(lo, hi);
                    }
                }
            }
        }
        // bias = -m (0 while nothing is visible) starts each score
        // accumulator, so a product's result is already the exponent; thr:
        // accumulator value above which m is raised
        float neg_m[HW], thr[HW];
        float thr_min = -INFINITY;                     // the smallest of thr
        f32x4_t bias[HW];
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
            neg_m[hh] = 0.f;
            thr[hh] = -INFINITY;
            bias[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        uint32_t kofs[KS];
        {
            const uint32_t kb0 = RB * j + 16 * (g ^ swz<D>(j));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kofs[ks] = kb0 ^ (64 * ks);
        }
        // K(t) operands from ring slot R
        auto load_kf = [&](auto rc, Frag8 (&kf)[KS][2]) {
            const uint8_t *base = slot_ptr(rc);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    kf[ks][kb].u = *reinterpret_cast<const uint4 *>(base + 16 * RB * kb + kofs[ks]);
            }
        };
        Frag8 kA[KS][2], kB[KS][2];                    // K operands of even / odd steps (t - t0)
        prologue();
        load_kf(int_c<0>{}, kA);
        uint32_t okw_cur = ok_bits(idx_of_step(t0));
        // first step whose keys cross the causal diagonal of this wave's first row
        const int s_diag = (qpos0 + 1) / TS;
        auto step = [&](auto rc, int t) -> bool {
            constexpr int R = decltype(rc)::value;
            constexpr int P = R & 1;
            const int32_t nix = idx_of_step(t + 1);
            if (t < t1w) {
                Frag8 (&kf)[KS][2] = (R & 1) ? kB : kA;  // read during step t-1
                Frag8 (&kn)[KS][2] = (R & 1) ? kA : kB;
                f32x4_t sc[HW][2];
                __builtin_amdgcn_s_setprio(3);         // the products of S(t) go first
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                        for (int hh = 0; hh < HW; ++hh)
                            sc[hh][kb] = mfma16(kf[ks][kb], qf[hh][ks], ks == 0 ? bias[hh] : sc[hh][kb]);
                    }
                }
                __builtin_amdgcn_s_setprio(0);
                // K(t+1) for the next step (its rows landed before the last
                // barrier), read while this step's vector work runs
                load_kf(int_c<(R + 1) % NB>{}, kn);
                const uint32_t okw = okw_cur;
                if (__builtin_expect(t >= s_diag || okw != 0xffffffffu, 0)) {
                    const int kb0 = TS * t;
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
                // One test for the 4 heads: the max of this lane's 32 scores
                // against the smallest threshold (a raise is needed only if
                // some head's max passes its own threshold, which implies this)
                float lmax;
                {
                    // (IEEE maximum: hipcc forms v_maximum3 from these nests)
                    auto max3 = [](float x, float y, float z) {
                        return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
                    };
                    float b[HW], c[HW];
#pragma unroll
                    for (int hh = 0; hh < HW; ++hh) {
                        const float a = max3(sc[hh][0][0], sc[hh][0][1], sc[hh][0][2]);
                        b[hh] = max3(sc[hh][0][3], sc[hh][1][0], sc[hh][1][1]);
                        c[hh] = max3(sc[hh][1][2], sc[hh][1][3], a);
                    }
                    const float m1 = max3(b[0], c[0], b[1]), m2 = max3(c[1], b[2], c[2]);
                    lmax = __builtin_elementwise_maximum(max3(b[3], c[3], m1), m2);
                }
                const uint64_t fire = __builtin_amdgcn_ballot_w64(lmax > thr_min);
                if (__builtin_expect(fire != 0, 0)) {
                    float lm[HW];
#pragma unroll
                    for (int hh = 0; hh < HW; ++hh)
                        lm[hh] = fmaxf(fmaxf(fmaxf(sc[hh][0][0], sc[hh][0][1]), fmaxf(sc[hh][0][2], sc[hh][0][3])),
                                       fmaxf(fmaxf(sc[hh][1][0], sc[hh][1][1]), fmaxf(sc[hh][1][2], sc[hh][1][3])));
                    // Raise the running max where a score exceeds it by more than
                    // kLazy (exact: the same stale max enters numerator and
                    // denominator, and probabilities stay below 2^8), and hand the
                    // factors to the output wave of these rows.
#pragma unroll
                    for (int hh = 0; hh < HW; ++hh) {
                        const float mx = max_over_groups(lm[hh]) - neg_m[hh];   // the row max
                        const float mnew = mx > m[hh] + kLazy ? mx : m[hh];
                        const float alpha = exp2_sub(m[hh], mnew);
                        {                              // in place: no copies on the common path
                            float x = m[hh];
                            // (alpha, computed from the old m, is an input: formed first)
                            asm volatile("v_mov_b32 %0, %1" : "+v"(x) : "v"(mnew), "v"(alpha));
                            m[hh] = x;
                        }
                        const float nb = mnew == -INFINITY ? 0.f : -mnew;
                        const float shift = nb - neg_m[hh];
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) sc[hh][kb] += shift;
                        neg_m[hh] = nb;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {          // in place: no copies on the common path
                            float x = bias[hh][r];
                            asm volatile("v_mov_b32 %0, %1" : "+v"(x) : "v"(nb));
                            bias[hh][r] = x;
                        }
                        thr[hh] = mnew == -INFINITY ? -INFINITY : kLazy;
                        if (g == 0) alpha_s[P][rb][hh][j] = alpha;
                    }
                    thr_min = fminf(fminf(thr[0], thr[1]), fminf(thr[2], thr[3]));
                    if (lane == 0) aflag[P][rb] = 1u;  // the output wave clears it after use
                }
#pragma unroll
                for (int hh = 0; hh < HW; ++hh) {
                    float p[2][4];
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) p[kb][r] = __builtin_amdgcn_exp2f(sc[hh][kb][r]);
                    }
                    uint4 w;
                    w.x = cvt_pk_bf16(p[0][0], p[0][1]);
                    w.y = cvt_pk_bf16(p[0][2], p[0][3]);
                    w.z = cvt_pk_bf16(p[1][0], p[1][1]);
                    w.w = cvt_pk_bf16(p[1][2], p[1][3]);
                    *reinterpret_cast<uint4 *>(p_addr(int_c<P>{}, hh)) = w;
                }
            }
            okw_cur = ok_bits(nix);
            phase_end();
            return t >= t1;
        };
        for (int t = t0;; t += NB) {
            if (step(int_c<0>{}, t)) break;
            if (step(int_c<1>{}, t + 1)) break;
            if (step(int_c<2>{}, t + 2)) break;
            if (step(int_c<3>{}, t + 3)) break;
            if (step(int_c<4>{}, t + 4)) break;
            if (step(int_c<5>{}, t + 5)) break;
        }
        wait_copies<0>();
        }
        // every copy into the ring has landed (each wave waited for its own):
        // the output waves stage their rows there (the output waves meet this
        // barrier at the same point)
        lds_barrier();
        if (pw < 0) return;
        // a split half: hand the running max to the output waves, then take
        // part in the publish / merge barriers (tid 0 keeps the count)
        int32_t *cnt = part_cnt + ps;
        if (g == 0) {
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) m_s[rb][hh][j] = m[hh];
        }
        if (tid == 0) seen = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (seen == 0) {
            __syncthreads();                           // the output waves' stores are complete
            if (tid == 0) seen = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (seen == 0) return;                     // the other half merges
        }
        if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // for the next call
        return;
    }
    // ================= output waves =================
    f32x4_t o[HW][DB], osum[HW];
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
        osum[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < DB; ++db) o[hh][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (t0 < t1) {
        Frag8 ones;
        ones.u = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
        pin(ones);                                     // a register, not rematerialised each step
        uint32_t vofs[DB];
        {
            const int vr = 4 * g + (j >> 2);
            const uint32_t vb0 = RB * vr + 8 * (j & 1) + 16 * (((j & 3) >> 1) ^ swz<D>(vr));
#pragma unroll
            for (int db = 0; db < DB; ++db) vofs[db] = vb0 ^ (32 * db);
        }
        prologue();
        auto step = [&](auto rc, int t) -> bool {
            constexpr int R = decltype(rc)::value;
            constexpr int R4 = (R + 4) % NB, RP = (R + NB - 1) % NB;   // ring slot of step t-1
            constexpr int P = (R + 1) & 1;                           // P slot of step t-1
            wait_copies<9>();                          // this wave's indices of step t+4
            int32_t sl4[2];
            slot_index(t + 4, sl4);
            if (t > t0 && t <= t1w) {
                // P(t-1) and V(t-1) (written / landed before the last barrier)
                const uint32_t fl = aflag[P][rb];
                Frag8 pf[HW], vf[DB];
#pragma unroll
                for (int hh = 0; hh < HW; ++hh) pf[hh].u = *reinterpret_cast<const uint4 *>(p_addr(int_c<P>{}, hh));
                const uint8_t *vbase = slot_ptr(int_c<RP>{}) + MAT;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    vf[db].h[0] = lds_read_tr16(reinterpret_cast<const uint16_t *>(vbase + vofs[db]));
                    vf[db].h[1] = lds_read_tr16(reinterpret_cast<const uint16_t *>(vbase + 16 * RB + vofs[db]));
                }
                if (__builtin_expect(__builtin_amdgcn_readfirstlane(static_cast<int>(fl)) != 0, 0)) {
                    if (lane == 0) aflag[P][rb] = 0u;  // read; the score wave sets it again two steps on at the earliest
#pragma unroll
                    for (int hh = 0; hh < HW; ++hh) {
                        const float a = alpha_s[P][rb][hh][j];
                        osum[hh] *= a;
#pragma unroll
                        for (int db = 0; db < DB; ++db) o[hh][db] *= a;
                    }
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
#pragma unroll
                    for (int hh = 0; hh < HW; ++hh) o[hh][db] = mfma16(vf[db], pf[hh], o[hh][db]);
                }
#pragma unroll
                for (int hh = 0; hh < HW; ++hh) osum[hh] = mfma16(ones, pf[hh], osum[hh]);
                pin(o);
                pin(osum);
            }
            fetch_idx(t + 6);
            issue(int_c<R4>{}, t + 4, sl4);
            wait_copies<10>();                         // rows of step t+2
            phase_end();
            return t >= t1;
        };
        for (int t = t0;; t += NB) {
            if (step(int_c<0>{}, t)) break;
            if (step(int_c<1>{}, t + 1)) break;
            if (step(int_c<2>{}, t + 2)) break;
            if (step(int_c<3>{}, t + 3)) break;
            if (step(int_c<4>{}, t + 4)) break;
            if (step(int_c<5>{}, t + 5)) break;
        }
        wait_copies<0>();
    }
    lds_barrier();                                     // the ring is idle (see the score waves)

    if (pw >= 0) {
        // One half of a split tile.  Each half leaves its unnormalised state
        // (O^T accumulators, running max m and row sum l of every row) in its
        // part of the workspace and counts itself done; the half that counts
        // second merges the other's state into its own and writes the output
        // (a row's softmax over both key sets: M = max(m, m'), weights
        // 2^(m - M) and 2^(m' - M) on the sums and accumulators).  The state
        // is written with agent-coherent stores, all complete before the
        // count (vector memory counter at zero), and read back with
        // agent-coherent loads issued after the count was seen, so the halves
        // may run on any two XCDs; no wave ever waits for another workgroup.
        // agent-coherent (sc1) buffer stores and loads over the two parts; a
        // part holds the O^T accumulators as [row block][head][column block]
        // [lane][4] (one 16-byte store per lane, a wave's covering 1 KB), then
        // (max, sum) as [row block][head][2][lane]
        constexpr uint32_t kAgent = 16;                // cache policy: scope bit sc1
        using u32x4_t = __attribute__((ext_vector_type(4))) unsigned int;
        const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
            part + (2 * ps + (pw & 1)) * kPart, 0, static_cast<int>(4 * kPart), 0x00020000);
        const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
            part + (2 * ps + ((pw & 1) ^ 1)) * kPart, 0, static_cast<int>(4 * kPart), 0x00020000);
        __syncthreads();                               // the running max and the count are in LDS
        float m[HW];
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) m[hh] = m_s[rb][hh][j];
        if (seen == 0) {
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    u32x4_t v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(o[hh][db][e]);
                    __builtin_amdgcn_raw_buffer_store_b128(v, mr, 16 * (((rb * HW + hh) * DB + db) * 64 + lane), 0,
                                                           kAgent);
                }
                const int ml = 4 * (kML + (rb * HW + hh) * 128 + lane);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m[hh]), mr, ml, 0, kAgent);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(osum[hh][0]), mr, ml + 256, 0, kAgent);
            }
            __builtin_amdgcn_s_waitcnt(0);             // every store of this wave is complete
            __syncthreads();                           // ... and of every wave
            __syncthreads();                           // the count is in LDS
            if (seen == 0) return;                     // the other half merges
        }
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
            const int ml = 4 * (kML + (rb * HW + hh) * 128 + lane);
            const float mo = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(orr, ml, 0, kAgent));
            const float lo = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(orr, ml + 256, 0, kAgent));
            const float mx = fmaxf(m[hh], mo);
            const float a = mx == -INFINITY ? 0.f : exp2_sub(m[hh], mx);
            const float b = mx == -INFINITY ? 0.f : exp2_sub(mo, mx);
            const float l = osum[hh][0] * a + lo * b;
            osum[hh] = f32x4_t{l, l, l, l};
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(
                    orr, 16 * (((rb * HW + hh) * DB + db) * 64 + lane), 0, kAgent);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[hh][db][e] = o[hh][db][e] * a + __uint_as_float(x[e]) * b;
            }
            __builtin_amdgcn_sched_barrier(0);         // one head's loads in flight at a time
        }
    }

    // The output rows.  A lane holds 4 consecutive d of one row, so storing
    // from the accumulators writes 16 rows 4 KB apart per instruction, 32
    // bytes each (the epilogue took ~3.5 us per workgroup).  Instead each
    // output wave stages its 16 rows, normalised and rounded, in its 16 KB of
    // the idle ring as 16 rows of 1 KB (the 4 heads side by side, as in out;
    // 16-byte chunks XOR-swizzled by row within each head), then stores one
    // whole row per instruction.
    {
        uint8_t *stage = ring + rb * (16 * HW * D * 2);
        static_assert(4 * 16 * HW * D * 2 <= NB * SLOT, "the staged rows fit in the ring");
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
            const float ls = osum[hh][0];
            const float inv = ls > 0.f ? 1.f / ls : 0.f;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                uint2 w;
                w.x = cvt_pk_bf16(o[hh][db][0] * inv, o[hh][db][1] * inv);
                w.y = cvt_pk_bf16(o[hh][db][2] * inv, o[hh][db][3] * inv);
                const int c = 2 * db + (g >> 1);       // 16-byte chunk of row j within head hh
                *reinterpret_cast<uint2 *>(stage + j * (HW * D * 2) + (hh * 16 + (c ^ j)) * 16 + 8 * (g & 1)) = w;
            }
        }
        wave_lds_fence();
        // row i: lane l stores bytes 16l .. 16l+15 of the row's 4 heads (chunk
        // l, staged at l ^ i)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (r0 + i < ti.rows) {
                const uint4 v = *reinterpret_cast<const uint4 *>(stage + i * (HW * D * 2) + (lane ^ i) * 16);
                *reinterpret_cast<uint4 *>(out + (static_cast<int64_t>(ti.q0 + ti.row0 + r0 + i) * n_heads + h0) * D + 8 * lane) = v;
            }
        }
    }
}

template <int G, bool WIDE>
hipError_t launch_rs(const PrefillArgs &a, hipStream_t s) {
    const int n = a.num_units > 0 ? a.num_units : a.num_q_tiles;
    const int64_t units = static_cast<int64_t>((n + kXcds - 1) / kXcds) * kXcds * a.pool.n_kv_heads * (G / 4);
    hipLaunchKernelGGL((prefill_rs_kernel<G, WIDE>), dim3(static_cast<unsigned>(units)), dim3(RsCfg::THREADS),
                       0, s, static_cast<const uint16_t *>(a.q), static_cast<uint16_t *>(a.out),
                       static_cast<const uint16_t *>(a.pool.k_layer),
                       static_cast<const uint16_t *>(a.pool.v_layer), a.pool.pool_slots,
                       a.pool.n_kv_heads, a.req_to_token, a.num_reqs, a.max_ctx_len, a.req_pool_indices,
                       a.qo_indptr, a.kv_indptr, a.q_tile_to_batch, a.q_tile_to_index, a.batch,
                       a.total_q, a.n_heads, a.num_q_tiles, a.scale_log2, a.units, a.num_units, a.num_pairs,
                       a.part_cnt, a.part);
    return hipGetLastError();
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

template <int D, int G, bool WIDE>
hipError_t launch_mfma(const PrefillArgs &a, hipStream_t s) {
    using C = MfmaCfg<D, G>;
    const int64_t units = static_cast<int64_t>((a.num_q_tiles + kXcds - 1) / kXcds) * kXcds *
                          a.pool.n_kv_heads * C::GROUPS;
    hipLaunchKernelGGL((prefill_mfma_kernel<D, G, WIDE>), dim3(static_cast<unsigned>(units)), dim3(C::THREADS),
                       0, s, static_cast<const uint16_t *>(a.q), static_cast<uint16_t *>(a.out),
                       static_cast<const uint16_t *>(a.pool.k_layer),
                       static_cast<const uint16_t *>(a.pool.v_layer), a.pool.pool_slots,
                       a.pool.n_kv_heads, a.req_to_token, a.num_reqs, a.max_ctx_len, a.req_pool_indices,
                       a.qo_indptr, a.kv_indptr, a.q_tile_to_batch, a.q_tile_to_index, a.batch,
                       a.total_q, a.n_heads, a.num_q_tiles, a.scale_log2);
    return hipGetLastError();
}

template <int D, bool WIDE>
hipError_t launch_mfma_g(const PrefillArgs &a, hipStream_t s) {
    if constexpr (D == 128) {
        switch (a.n_heads / a.pool.n_kv_heads) {
            case 4: return launch_rs<4, WIDE>(a, s);
            case 8: return launch_rs<8, WIDE>(a, s);
            default: break;
        }
    }
    switch (a.n_heads / a.pool.n_kv_heads) {
        case 1: return launch_mfma<D, 1, WIDE>(a, s);
        case 2: return launch_mfma<D, 2, WIDE>(a, s);
        case 4: return launch_mfma<D, 4, WIDE>(a, s);
        case 6: return launch_mfma<D, 6, WIDE>(a, s);
        case 8: return launch_mfma<D, 8, WIDE>(a, s);
        default: return hipErrorInvalidValue;
    }
}

// Slots wider than a buffer record stride can express (16383 bytes) are
// addressed as (slot, KV head) rows.
template <int D>
hipError_t launch_mfma_d(const PrefillArgs &a, hipStream_t s) {
    return static_cast<int64_t>(a.pool.n_kv_heads) * D * 2 > kMaxRecordStride ? launch_mfma_g<D, true>(a, s)
                                                                             : launch_mfma_g<D, false>(a, s);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
    if (a.num_q_tiles == 0) return hipSuccess;
    if (a.pool.dtype == 1)
        return a.pool.head_dim == 128 ? launch_mfma_d<128>(a, s) : launch_mfma_d<64>(a, s);
    return a.pool.head_dim == 128 ? launch_generic<float, 128>(a, s) : launch_generic<float, 64>(a, s);
}

}  // namespace astr
