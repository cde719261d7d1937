// The C entry points of libastr: argument validation, then one launcher call
// on the caller's stream.  Nothing here allocates, frees or synchronises
// device memory, and no call switches to another implementation when a shape
// or dtype is unsupported -- it returns an error instead.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>

#include "astr.h"
#include "astr_ceiling.h"
#include "kernels.hpp"
#include "status.hpp"

namespace astr {

namespace {
thread_local char g_err[512] = "";
}

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

namespace {

constexpr double kLog2e = 1.4426950408889634074;

bool group_supported(int g) { return g == 1 || g == 2 || g == 4 || g == 6 || g == 8; }

// Checks shared by every attention-side call; fills the layer view.
int check_pool(const char *who, const astr_kv_meta *m, int n_heads, int layer_id, PoolView &pv) {
    if (!m) return fail(ASTR_E_INVAL, "%s: null meta", who);
    if (m->kv_dtype != ASTR_F32 && m->kv_dtype != ASTR_BF16)
        return fail(ASTR_E_UNSUPPORTED, "%s: kv_dtype %d (supported: f32, bf16)", who, m->kv_dtype);
    if (m->head_dim != 64 && m->head_dim != 128)
        return fail(ASTR_E_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", who, m->head_dim);
    if (m->n_kv_heads < 1 || n_heads < 1 || n_heads % m->n_kv_heads != 0)
        return fail(ASTR_E_INVAL, "%s: n_heads %d is not a multiple of n_kv_heads %d", who, n_heads,
                    m->n_kv_heads);
    if (!group_supported(n_heads / m->n_kv_heads))
        return fail(ASTR_E_UNSUPPORTED, "%s: %d query heads per KV head (supported: 1, 2, 4, 6, 8)", who,
                    n_heads / m->n_kv_heads);
    if (m->n_kv_heads > 65535) return fail(ASTR_E_UNSUPPORTED, "%s: too many KV heads", who);
    if (!m->k_buffer || !m->v_buffer || m->pool_slots < 1 || m->n_layers < 1)
        return fail(ASTR_E_INVAL, "%s: empty pool", who);
    if (layer_id < 0 || layer_id >= m->n_layers)
        return fail(ASTR_E_INVAL, "%s: layer_id %d outside [0, %d)", who, layer_id, m->n_layers);
    const size_t esz = m->kv_dtype == ASTR_BF16 ? 2 : 4;
    const size_t layer_bytes = static_cast<size_t>(m->pool_slots) * m->n_kv_heads * m->head_dim * esz;
    pv.k_layer = static_cast<char *>(m->k_buffer) + layer_bytes * layer_id;
    pv.v_layer = static_cast<char *>(m->v_buffer) + layer_bytes * layer_id;
    pv.pool_slots = m->pool_slots;
    pv.n_kv_heads = m->n_kv_heads;
    pv.head_dim = m->head_dim;
    pv.dtype = m->kv_dtype;
    return ASTR_OK;
}

// Activations (q, k, v, out) are stored in the pool's dtype: the kernels
// read and write them with the pool's element type.
int check_act(const char *who, const astr_kv_meta *m, int act_dtype) {
    if (act_dtype != ASTR_F32 && act_dtype != ASTR_BF16)
        return fail(ASTR_E_UNSUPPORTED, "%s: act_dtype %d (supported: f32, bf16)", who, act_dtype);
    if (act_dtype != m->kv_dtype)
        return fail(ASTR_E_UNSUPPORTED, "%s: act_dtype %d differs from kv_dtype %d (activations use the pool's dtype)",
                    who, act_dtype, m->kv_dtype);
    return ASTR_OK;
}

int check_table(const char *who, const astr_kv_meta *m) {
    if (m->batch < 0) return fail(ASTR_E_INVAL, "%s: batch %d", who, m->batch);
    if (m->batch == 0) return ASTR_OK;
    if (!m->req_to_token || !m->req_pool_indices || !m->kv_indptr || m->num_reqs < 1 ||
        m->max_ctx_len < 1)
        return fail(ASTR_E_INVAL, "%s: missing request table", who);
    if (m->max_len < 0 || m->max_len > m->max_ctx_len)
        return fail(ASTR_E_INVAL, "%s: max_len %d outside [0, max_ctx_len %d]", who, m->max_len,
                    m->max_ctx_len);
    return ASTR_OK;
}

int launched(const char *who, hipError_t e) {
    if (e != hipSuccess) return fail(ASTR_E_LAUNCH, "%s: %s", who, hipGetErrorString(e));
    return ASTR_OK;
}

float scale_of(float sm_scale, int head_dim) {
    const double s = sm_scale > 0.f ? static_cast<double>(sm_scale) : 1.0 / std::sqrt(static_cast<double>(head_dim));
    return static_cast<float>(s * kLog2e);
}

}  // namespace
}  // namespace astr

using astr::fail;

extern "C" const char *astr_last_error(void) { return astr::g_err; }

extern "C" int astr_rope_table(float *freqs_cis, int max_pos, int head_dim, double theta, void *stream) {
    if (!freqs_cis || max_pos < 1 || head_dim < 2 || head_dim % 2 || !(theta > 1.0))
        return fail(ASTR_E_INVAL, "rope_table: bad argument");
    return astr::launched("rope_table",
                          astr::launch_rope_table(freqs_cis, max_pos, head_dim, theta,
                                                  static_cast<hipStream_t>(stream)));
}

extern "C" int astr_rope_kv_write(void *q, const void *k, const void *v, const int32_t *positions,
                                  const int32_t *out_cache_loc, int n_tokens, int n_heads,
                                  const float *freqs_cis, int max_pos, const astr_kv_meta *m,
                                  int layer_id, astr_dtype act_dtype, void *stream) {
    astr::RopeArgs a{};
    int st = astr::check_pool("rope_kv_write", m, n_heads, layer_id, a.pool);
    if (st) return st;
    st = astr::check_act("rope_kv_write", m, act_dtype);
    if (st) return st;
    if (n_tokens < 0) return fail(ASTR_E_INVAL, "rope_kv_write: n_tokens %d", n_tokens);
    if (n_tokens == 0) return ASTR_OK;
    if (!q || !k || !v || !positions || !out_cache_loc || !freqs_cis || max_pos < 1)
        return fail(ASTR_E_INVAL, "rope_kv_write: null argument or max_pos < 1");
    a.q = q;
    a.k = k;
    a.v = v;
    a.positions = positions;
    a.out_cache_loc = out_cache_loc;
    a.n_tokens = n_tokens;
    a.n_heads = n_heads;
    a.freqs = freqs_cis;
    a.max_pos = max_pos;
    return astr::launched("rope_kv_write", astr::launch_rope_kv_write(a, static_cast<hipStream_t>(stream)));
}

extern "C" int astr_rope_backward(void *grad, const int32_t *positions, int n_tokens, int n_heads,
                                  int head_dim, const float *freqs_cis, int max_pos, astr_dtype dtype,
                                  void *stream) {
    if (n_tokens < 0 || n_heads < 1) return fail(ASTR_E_INVAL, "rope_backward: n_tokens %d, n_heads %d", n_tokens, n_heads);
    if (dtype != ASTR_F32 && dtype != ASTR_BF16) return fail(ASTR_E_UNSUPPORTED, "rope_backward: dtype %d", dtype);
    if (head_dim != 64 && head_dim != 128)
        return fail(ASTR_E_UNSUPPORTED, "rope_backward: head_dim %d (supported: 64, 128)", head_dim);
    if (n_tokens == 0) return ASTR_OK;
    if (!grad || !positions || !freqs_cis || max_pos < 1)
        return fail(ASTR_E_INVAL, "rope_backward: null argument or max_pos < 1");
    if (static_cast<int64_t>(n_tokens) * n_heads * head_dim / 4 > static_cast<int64_t>(UINT32_MAX) * 256)
        return fail(ASTR_E_UNSUPPORTED, "rope_backward: too many elements");
    return astr::launched("rope_backward",
                          astr::launch_rope_backward(grad, positions, n_tokens, n_heads, head_dim, dtype,
                                                     freqs_cis, max_pos, static_cast<hipStream_t>(stream)));
}

extern "C" int astr_decode_num_splits(int max_len, int split_chunk) {
    if (max_len < 0 || split_chunk < 1) return 0;
    const int s = (max_len + split_chunk - 1) / split_chunk;
    return s < 1 ? 1 : s;
}

extern "C" size_t astr_decode_workspace_bytes(int batch, int n_heads, int head_dim, int max_len, int split_chunk) {
    if (batch < 0 || n_heads < 1 || head_dim < 1 || max_len < 0 || split_chunk < 1) return 0;
    const int s = astr_decode_num_splits(max_len, split_chunk);
    if (s <= 1) return 0;                              // one split: the output is written directly
    const size_t rows = static_cast<size_t>(batch) * n_heads * s;
    return rows * static_cast<size_t>(head_dim) * 4 + rows * 4;
}

namespace {
// Shared by the plain and the fused decode call: validation and arguments.
int decode_args(const char *what, const void *q, void *out, int n_heads, const astr_kv_meta *m,
                int layer_id, int split_chunk, float sm_scale, float *o_part, float *lse_part,
                int act_dtype, astr::DecodeArgs &a, bool &empty) {
    empty = false;
    int st = astr::check_pool(what, m, n_heads, layer_id, a.pool);
    if (st) return st;
    st = astr::check_act(what, m, act_dtype);
    if (st) return st;
    st = astr::check_table(what, m);
    if (st) return st;
    if (m->batch == 0) {
        empty = true;
        return ASTR_OK;
    }
    if (!q || !out) return fail(ASTR_E_INVAL, "%s: null q or out", what);
    if (split_chunk < 1) return fail(ASTR_E_INVAL, "%s: split_chunk %d", what, split_chunk);
    const int ns = astr_decode_num_splits(m->max_len, split_chunk);
    if (ns > 1 && (!o_part || !lse_part))
        return fail(ASTR_E_INVAL, "%s: %d splits need o_part and lse_part", what, ns);
    if (static_cast<int64_t>(m->batch) * ns * m->n_kv_heads > INT32_MAX)
        return fail(ASTR_E_UNSUPPORTED, "%s: grid too large", what);
    if (m->split_item_batch || m->split_item_index || m->num_split_items) {
        if (!m->split_item_batch || !m->split_item_index || m->num_split_items < 1)
            return fail(ASTR_E_INVAL, "%s: incomplete decode work items", what);
        if (m->split_item_chunk != split_chunk)
            return fail(ASTR_E_INVAL, "%s: work items built for split_chunk %d, called with %d", what,
                        m->split_item_chunk, split_chunk);
        if (static_cast<int64_t>(m->num_split_items) * m->n_kv_heads > INT32_MAX)
            return fail(ASTR_E_UNSUPPORTED, "%s: grid too large", what);
        a.item_batch = m->split_item_batch;
        a.item_index = m->split_item_index;
        a.num_items = m->num_split_items;
    }
    a.q = q;
    a.out = out;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.req_to_token = m->req_to_token;
    a.num_reqs = m->num_reqs;
    a.max_ctx_len = m->max_ctx_len;
    a.req_pool_indices = m->req_pool_indices;
    a.kv_indptr = m->kv_indptr;
    a.batch = m->batch;
    a.n_heads = n_heads;
    a.split_chunk = split_chunk;
    a.n_splits = ns;
    a.scale_log2 = astr::scale_of(sm_scale, m->head_dim);
    return ASTR_OK;
}
}  // namespace

extern "C" int astr_decode_attn(const void *q, int n_heads, const astr_kv_meta *m, int layer_id,
                                int split_chunk, float sm_scale, float *o_part, float *lse_part, void *out,
                                astr_dtype act_dtype, void *stream) {
    astr::DecodeArgs a{};
    bool empty;
    const int st = decode_args("decode_attn", q, out, n_heads, m, layer_id, split_chunk, sm_scale, o_part,
                               lse_part, act_dtype, a, empty);
    if (st || empty) return st;
    return astr::launched("decode_attn", astr::launch_decode(a, static_cast<hipStream_t>(stream)));
}

static_assert(astr::kStaticDecodeScratchBytes == ASTR_DECODE_STATIC_SCRATCH_BYTES,
              "the header states the static scratch size");

extern "C" int astr_decode_attn_noalloc(const void *q, int n_heads, const astr_kv_meta *m, int layer_id,
                                        int split_chunk, float sm_scale, void *out, astr_dtype act_dtype,
                                        void *stream) {
    if (!m) return fail(ASTR_E_INVAL, "decode_attn_noalloc: null meta");
    float *o_part = nullptr, *lse_part = nullptr;
    const size_t need = astr_decode_workspace_bytes(m->batch, n_heads, m->head_dim, m->max_len, split_chunk);
    if (need > astr::kStaticDecodeScratchBytes)
        return fail(ASTR_E_INVAL,
                    "decode_attn_noalloc: the split-K scratch needs %zu bytes, the static scratch holds %zu "
                    "(use astr_decode_attn with a caller-owned workspace, or a larger split_chunk)",
                    need, astr::kStaticDecodeScratchBytes);
    if (need > 0) {
        const hipError_t e = astr::static_decode_scratch(&o_part);
        if (e != hipSuccess)
            return fail(ASTR_E_LAUNCH, "decode_attn_noalloc: static scratch: %s", hipGetErrorString(e));
        const size_t rows = static_cast<size_t>(m->batch) * n_heads *
                            astr_decode_num_splits(m->max_len, split_chunk);
        lse_part = o_part + rows * m->head_dim;
    }
    astr::DecodeArgs a{};
    bool empty;
    const int st = decode_args("decode_attn_noalloc", q, out, n_heads, m, layer_id, split_chunk, sm_scale, o_part,
                               lse_part, act_dtype, a, empty);
    if (st || empty) return st;
    return astr::launched("decode_attn_noalloc", astr::launch_decode(a, static_cast<hipStream_t>(stream)));
}

extern "C" int astr_decode_attn_write(const void *q, const void *k_new, const void *v_new, int n_heads,
                                      const astr_kv_meta *m, int layer_id, const float *freqs_cis, int max_pos,
                                      int split_chunk, float sm_scale, float *o_part, float *lse_part,
                                      void *out, astr_dtype act_dtype, void *stream) {
    astr::DecodeArgs a{};
    bool empty;
    const int st = decode_args("decode_attn_write", q, out, n_heads, m, layer_id, split_chunk, sm_scale,
                               o_part, lse_part, act_dtype, a, empty);
    if (st || empty) return st;
    if (m->kv_dtype != ASTR_BF16)
        return fail(ASTR_E_UNSUPPORTED, "decode_attn_write: bf16 only (use astr_rope_kv_write + astr_decode_attn)");
    if (!k_new || !v_new || !freqs_cis) return fail(ASTR_E_INVAL, "decode_attn_write: null k_new, v_new or freqs_cis");
    if (max_pos < m->max_len)
        return fail(ASTR_E_INVAL, "decode_attn_write: max_pos %d < max_len %d", max_pos, m->max_len);
    a.k_new = k_new;
    a.v_new = v_new;
    a.freqs = freqs_cis;
    a.max_pos = max_pos;
    return astr::launched("decode_attn_write", astr::launch_decode(a, static_cast<hipStream_t>(stream)));
}

extern "C" int astr_prefill_attn(const void *q, int total_q, int n_heads, const astr_kv_meta *m,
                                 int layer_id, float sm_scale, void *out, astr_dtype act_dtype, void *stream) {
    astr::PrefillArgs a{};
    int st = astr::check_pool("prefill_attn", m, n_heads, layer_id, a.pool);
    if (st) return st;
    st = astr::check_act("prefill_attn", m, act_dtype);
    if (st) return st;
    st = astr::check_table("prefill_attn", m);
    if (st) return st;
    if (m->batch == 0 || m->num_q_tiles == 0) return ASTR_OK;
    if (m->num_q_tiles < 0) return fail(ASTR_E_INVAL, "prefill_attn: num_q_tiles %d", m->num_q_tiles);
    if (m->q_tile != 64) return fail(ASTR_E_UNSUPPORTED, "prefill_attn: q_tile %d (supported: 64)", m->q_tile);
    if (!q || !out || !m->qo_indptr || !m->q_tile_to_batch || !m->q_tile_to_index)
        return fail(ASTR_E_INVAL, "prefill_attn: null q, out or tile metadata");
    if (n_heads > 65535) return fail(ASTR_E_UNSUPPORTED, "prefill_attn: too many heads");
    if (total_q < 0) return fail(ASTR_E_INVAL, "prefill_attn: total_q %d", total_q);
    // bf16: slots wider than a buffer record are addressed as (slot, KV head)
    // records, whose index must fit 32 bits
    if (m->kv_dtype == ASTR_BF16 && static_cast<int64_t>(m->n_kv_heads) * m->head_dim * 2 > astr::kMaxRecordStride &&
        m->pool_slots * m->n_kv_heads > static_cast<int64_t>(UINT32_MAX))
        return fail(ASTR_E_UNSUPPORTED, "prefill_attn: pool_slots * n_kv_heads exceeds 2^32 - 1");
    a.q = q;
    a.total_q = total_q;
    a.out = out;
    a.req_to_token = m->req_to_token;
    a.num_reqs = m->num_reqs;
    a.max_ctx_len = m->max_ctx_len;
    a.req_pool_indices = m->req_pool_indices;
    a.qo_indptr = m->qo_indptr;
    a.kv_indptr = m->kv_indptr;
    a.q_tile_to_batch = m->q_tile_to_batch;
    a.q_tile_to_index = m->q_tile_to_index;
    a.batch = m->batch;
    a.num_q_tiles = m->num_q_tiles;
    a.q_tile = m->q_tile;
    a.n_heads = n_heads;
    a.scale_log2 = astr::scale_of(sm_scale, m->head_dim);
    if (m->prefill_units || m->num_prefill_units || m->num_prefill_pairs) {
        if (!m->prefill_units || m->num_prefill_units < 1 || m->num_prefill_pairs < 0)
            return fail(ASTR_E_INVAL, "prefill_attn: incomplete work plan");
        if (m->num_prefill_pairs > m->num_prefill_units / 2)
            return fail(ASTR_E_INVAL, "prefill_attn: %d split tiles need %d units, the plan has %d",
                        m->num_prefill_pairs, 2 * m->num_prefill_pairs, m->num_prefill_units);
        if (reinterpret_cast<uintptr_t>(m->prefill_units) % 16 != 0)
            return fail(ASTR_E_INVAL, "prefill_attn: work plan units not 16-byte aligned");
        if (m->num_prefill_pairs > 0 && !m->prefill_workspace)
            return fail(ASTR_E_INVAL, "prefill_attn: a plan with %d split tiles needs a workspace",
                        m->num_prefill_pairs);
        if (m->num_prefill_units > 16 * static_cast<int64_t>(m->num_q_tiles) ||
            static_cast<int64_t>(m->num_prefill_units) * m->n_kv_heads * ((n_heads / m->n_kv_heads + 3) / 4) +
                    8 * 64 > INT32_MAX ||
            astr::prefill_part_slots(m->num_prefill_pairs, n_heads) * 2 * astr::kPrefillPartFloats >
                INT64_MAX / 8)
            return fail(ASTR_E_INVAL, "prefill_attn: work plan too large for %d tiles", m->num_q_tiles);
        if (m->num_prefill_pairs > 0 &&
            m->prefill_workspace_bytes < astr_prefill_workspace_bytes(m->num_prefill_pairs, n_heads, m->head_dim))
            return fail(ASTR_E_INVAL, "prefill_attn: workspace of %zu bytes, the plan needs %zu",
                        m->prefill_workspace_bytes,
                        astr_prefill_workspace_bytes(m->num_prefill_pairs, n_heads, m->head_dim));
        a.units = m->prefill_units;
        a.num_units = m->num_prefill_units;
        a.num_pairs = m->num_prefill_pairs;
        const int64_t slots = astr::prefill_part_slots(m->num_prefill_pairs, n_heads);
        a.part_cnt = static_cast<int32_t *>(m->prefill_workspace);
        a.part = m->num_prefill_pairs > 0
                     ? reinterpret_cast<float *>(static_cast<char *>(m->prefill_workspace) +
                                                 astr::prefill_counts_bytes(slots))
                     : nullptr;
    }
    return astr::launched("prefill_attn", astr::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

extern "C" size_t astr_prefill_workspace_bytes(int pairs, int n_heads, int head_dim) {
    if (pairs < 0 || n_heads < 1 || head_dim < 1) return 0;
    if (pairs == 0) return 0;
    const int64_t slots = astr::prefill_part_slots(pairs, n_heads);
    return static_cast<size_t>(astr::prefill_counts_bytes(slots) + slots * 2 * astr::kPrefillPartFloats * 4);
}

extern "C" int astr_ceiling_stream_read(const void *buf, size_t bytes, int workgroups, int nontemporal,
                                        uint32_t *sink, void *stream) {
    if (!buf || !sink || workgroups < 1 || bytes < 16 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(buf) % 16 != 0)
        return fail(ASTR_E_INVAL, "ceiling_stream_read: bad argument");
    return astr::launched("ceiling_stream_read",
                          astr::launch_ceiling_stream_read(buf, bytes, workgroups, nontemporal != 0, sink,
                                                           static_cast<hipStream_t>(stream)));
}

extern "C" int astr_ceiling_mfma_loop(int workgroups, int iters, float *sink, void *stream) {
    if (!sink || workgroups < 1 || iters < 1) return fail(ASTR_E_INVAL, "ceiling_mfma_loop: bad argument");
    return astr::launched("ceiling_mfma_loop",
                          astr::launch_ceiling_mfma_loop(workgroups, iters, sink, static_cast<hipStream_t>(stream)));
}
