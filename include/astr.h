/*
 * astr.h -- C ABI of the paged grouped-query attention library for AMD
 * MI355X (gfx950): rotary embedding fused with the KV-cache write, split-K
 * paged decode attention with its log-sum-exp merge, ragged causal prefill
 * attention over a paged pool, and the host-side page-table builder.
 *
 * Definitions followed (AstrAI documentation pages):
 *   docs/developer/internals.md -- "Autoregression & Causal Masking",
 *     "Rotary Position Embedding (RoPE)", "KV Cache Mathematics",
 *     "Cache Architecture", "Attention Backend".
 *   docs/guides/inference.md -- "KV Cache", "KVCache System",
 *     "Attention Backend", "Rotary Embedding Backend".
 *   AstrAI paper (main.tex) -- "Model Architecture" (GQA, RoPE theta 10 000).
 *
 * Conventions shared by every call
 *   - Device pointers point to memory the caller owns (in practice PyTorch
 *     tensors).  The library never allocates, frees or synchronises device
 *     memory; every device call is enqueued on the caller's stream and
 *     returns without waiting.  `stream` is a hipStream_t (NULL = the
 *     default stream).
 *   - Host pointers are read during the call only, except where stated.
 *   - Every argument is validated on the host before anything is launched.
 *     On a non-OK return nothing was enqueued and astr_last_error() gives a
 *     message.  An unsupported dtype or head_dim is an error, never a silent
 *     switch to another implementation (inference.md, "Attention Backend":
 *     the kernel wrappers raise instead of falling back, and an explicit
 *     selection fails rather than switching).
 *   - Indices read from device metadata are bounds-checked in the kernels:
 *     a slot outside [0, pool_slots) or a position outside [0, max_pos) is
 *     skipped (it is neither read nor written), so malformed metadata cannot
 *     make a kernel touch memory outside the buffers it was given.
 *   - Layouts are row-major.  q/k/v are [tokens, heads, head_dim] ("blhd"
 *     with the batch and sequence axes flattened, internals.md "Attention
 *     Backend"); query head h reads KV head h / (n_heads / n_kv_heads).
 *   - Supported: kv_dtype in {ASTR_F32, ASTR_BF16}; head_dim in {64, 128};
 *     n_heads / n_kv_heads in {1, 2, 4, 6, 8} (one compiled kernel per
 *     group size; any other divisor returns ASTR_E_UNSUPPORTED).  The
 *     device calls take the activations' dtype (act_dtype: q, k, v, out);
 *     it must equal the pool's kv_dtype, else ASTR_E_UNSUPPORTED.
 *     Accumulation is float32.
 */
#ifndef ASTR_H
#define ASTR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum astr_status {
    ASTR_OK = 0,
    ASTR_E_INVAL = -1,        /* bad argument: null pointer, size or index out of range */
    ASTR_E_UNSUPPORTED = -2,  /* well-formed but not implemented (dtype, head_dim, group) */
    ASTR_E_NOMEM = -3,        /* page pool or request slots exhausted; state unchanged */
    ASTR_E_LAUNCH = -4        /* the HIP runtime rejected a kernel launch */
} astr_status;

typedef enum astr_dtype { ASTR_F32 = 0, ASTR_BF16 = 1 } astr_dtype;

/*
 * The per-step view of the KV cache handed to the attention calls: the
 * fields of the KVCache record (inference.md, "KVCache System").  Pointers
 * are device pointers; the scalar sizes are host values, so that no call
 * needs a device-to-host read (max_len is kept on the host for that reason).
 */
typedef struct astr_kv_meta {
    void *k_buffer;                   /* [n_layers, pool_slots, n_kv_heads, head_dim] kv_dtype */
    void *v_buffer;                   /* same shape and dtype */
    int64_t pool_slots;               /* token slots per layer */
    int32_t n_layers;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t kv_dtype;                 /* astr_dtype */
    const int32_t *req_to_token;      /* [num_reqs, max_ctx_len]: (request, position) -> slot */
    int32_t num_reqs;
    int32_t max_ctx_len;              /* row stride of req_to_token */
    const int32_t *req_pool_indices;  /* [batch]: request row of each batch entry */
    const int32_t *kv_indptr;         /* [batch + 1]: prefix sum of KV lengths (seq_lens) */
    const int32_t *qo_indptr;         /* [batch + 1]: prefix sum of query lengths (prefill) */
    const int32_t *q_tile_to_batch;   /* [num_q_tiles]: query tile -> batch entry (prefill) */
    const int32_t *q_tile_to_index;   /* [num_q_tiles]: query tile -> tile index in its request */
    int32_t batch;                    /* host: number of requests in the step */
    int32_t max_len;                  /* host: max KV length over the batch */
    int32_t num_q_tiles;              /* host (prefill) */
    int32_t q_tile;                   /* host (prefill): query rows per tile */
    /* Decode work items (optional).  When set, the decode calls launch one
     * workgroup per (item, KV head) instead of one per (batch entry, split
     * index below ceil(max_len / split_chunk)), most of which would find
     * their split past the request's end and exit without work.  Built by
     * astr_decode_split_items for the split_chunk of the call. */
    const int32_t *split_item_batch;  /* [num_split_items]: batch entry of each item */
    const int32_t *split_item_index;  /* [num_split_items]: split index of each item */
    int32_t num_split_items;          /* host: 0 = no item list */
    int32_t split_item_chunk;         /* host: split_chunk the items were built for */
    /* Prefill work plan (optional; built by astr_prefill_plan).  A unit is a
     * query tile's key steps [step_lo, step_hi) (steps of 32 keys; step_hi is
     * clamped to the tile's last step).  When set, the bf16 prefill with
     * head_dim 128 and a multiple of 4 query heads per KV head launches one
     * workgroup per (unit, KV head, group of 4 query heads), in unit order;
     * other configurations ignore the plan.  The two units of a split tile
     * (a pair) each leave their unnormalised partial result in the
     * workspace, and the one that finishes second merges both.  16-byte
     * aligned device array. */
    const int32_t *prefill_units;     /* [num_prefill_units][8]: tile, step_lo, step_hi,
                                         2 * pair + (0 lower keys, 1 upper keys) or -1,
                                         then the tile's request row, first query row,
                                         rows (0: nothing to do) and first row's position */
    int32_t num_prefill_units;        /* host: 0 = one unit per tile, in tile order */
    int32_t num_prefill_pairs;        /* host: split tiles in the plan */
    void *prefill_workspace;          /* device, zeroed before its first use */
    size_t prefill_workspace_bytes;   /* host: its size, >= astr_prefill_workspace_bytes(
                                         num_prefill_pairs, n_heads, head_dim) */
} astr_kv_meta;

/* Message for the last non-OK status returned on the calling thread. */
const char *astr_last_error(void);

/* ------------------------------------------------------------------------ */
/* Rotary embedding                                                         */
/* ------------------------------------------------------------------------ */

/*
 * Fill the rotary cos/sin table (internals.md, "Rotary Position Embedding":
 * freqs_cis of shape [max_len, dim/2, 2], float32 [cos, sin] pairs).
 * Entry [pos, i] = (cos(pos * w_i), sin(pos * w_i)) with w_i = theta^(-2i/head_dim)
 * (RoFormer frequencies, theta from the paper's "Model Architecture" table);
 * the angle and both functions are evaluated in float64 and rounded to float32.
 *   freqs_cis  device, [max_pos, head_dim/2, 2] float32, written.
 * Errors: INVAL (null, max_pos < 1, odd or non-positive head_dim, theta <= 1).
 */
int astr_rope_table(float *freqs_cis, int max_pos, int head_dim, double theta, void *stream);

/*
 * Rotate q and k by their token's position, then write the rotated k and the
 * unrotated v into the pool row out_cache_loc[t] of layer layer_id:
 *   k_buffer[layer_id, out_cache_loc[t], h, :] = R(positions[t]) k[t, h, :]
 *   v_buffer[layer_id, out_cache_loc[t], h, :] = v[t, h, :]
 *   q[t, h, :] <- R(positions[t]) q[t, h, :]            (in place)
 * RoPE is applied before the cache write (internals.md, "KV Cache
 * Mathematics": cached keys keep the rotation of their own position;
 * inference.md, "KV Cache").  R rotates each adjacent pair (x[2i], x[2i+1])
 * as the complex product with freqs_cis[pos, i] (inference.md, "Rotary
 * Embedding Backend": view as complex, multiply, view as real).  The product
 * is evaluated in float64 from the float32 table entries (so each result is
 * the correctly rounded rotation by the table) and rounded once to the
 * storage type; bf16 rounds to nearest-even.
 *   q              device [n_tokens, n_heads, head_dim] kv_dtype, read and written
 *   k, v           device [n_tokens, m->n_kv_heads, head_dim] kv_dtype, read
 *   positions      device [n_tokens] int32, position of each token
 *   out_cache_loc  device [n_tokens] int32, destination slot of each token
 *   freqs_cis      device [max_pos, head_dim/2, 2] float32 (astr_rope_table)
 *   m              host; uses k_buffer, v_buffer, pool_slots, n_layers,
 *                  n_kv_heads, head_dim, kv_dtype
 *   act_dtype      dtype of q, k and v; must equal m->kv_dtype
 * n_tokens == 0 is a no-op.  Tokens whose slot or position is out of range are
 * skipped entirely.  Errors: INVAL, UNSUPPORTED, LAUNCH.
 */
int astr_rope_kv_write(void *q, const void *k, const void *v,
                       const int32_t *positions, const int32_t *out_cache_loc,
                       int n_tokens, int n_heads, const float *freqs_cis, int max_pos,
                       const astr_kv_meta *m, int layer_id, astr_dtype act_dtype, void *stream);

/*
 * Gradient of the rotation (the backward pass of the rotary embedding used in
 * training: internals.md, "Rotary Position Embedding (RoPE)" and
 * inference.md, "Rotary Embedding Backend" keep the complex-multiply path for
 * autograd).  The rotation by freqs_cis[pos] is linear, so the gradient with
 * respect to its input is its transpose applied to the gradient of its output:
 *   grad[t, h, :] <- R(positions[t])^T grad[t, h, :]        (in place)
 * i.e. each adjacent pair times the complex conjugate of the same table entry
 * the forward used.  Evaluated in float64 from the float32 entries, rounded
 * once to dtype (bf16: nearest-even).
 *   grad       device [n_tokens, n_heads, head_dim] dtype, read and written
 *   positions  device [n_tokens] int32
 *   freqs_cis  device [max_pos, head_dim/2, 2] float32 (astr_rope_table)
 * n_tokens == 0 is a no-op; tokens whose position is outside [0, max_pos) are
 * left unchanged.  Errors: INVAL, UNSUPPORTED (dtype, head_dim 64/128 only),
 * LAUNCH.
 */
int astr_rope_backward(void *grad, const int32_t *positions, int n_tokens, int n_heads, int head_dim,
                       const float *freqs_cis, int max_pos, astr_dtype dtype, void *stream);

/* ------------------------------------------------------------------------ */
/* Decode attention (one query token per request)                          */
/* ------------------------------------------------------------------------ */

/* Number of KV splits S = ceil(max_len / split_chunk) (0 on bad input). */
int astr_decode_num_splits(int max_len, int split_chunk);

/*
 * Bytes of the split-K scratch of one decode call: the partial outputs and
 * log-sum-exps of every (request, query head, split), the decode_o_part and
 * decode_ml_part buffers of the KVCache record (inference.md, "KVCache
 * System") with the split axis made explicit.  With S = ceil(max_len /
 * split_chunk) and R = batch * n_heads * S the scratch is
 *   o_part    float32 [batch, n_heads, S, head_dim]  (R * head_dim * 4 bytes)
 *   lse_part  float32 [batch, n_heads, S]            (R * 4 bytes)
 * and the value returned is their sum, so that one allocation can hold both
 * (o_part first, lse_part at byte R * head_dim * 4, a multiple of 16).  0
 * when S <= 1 (the decode then writes its output directly and touches no
 * scratch) and on bad input (batch < 0, n_heads < 1, head_dim < 1,
 * max_len < 0, split_chunk < 1).
 */
size_t astr_decode_workspace_bytes(int batch, int n_heads, int head_dim, int max_len, int split_chunk);
/*
 * The decode work items of a step (host only): for each batch entry b the
 * splits s < max(1, ceil(seq_lens[b] / split_chunk)) -- every (request,
 * split) that holds keys, the partials of the KVCache record's
 * decode_o_part / decode_ml_part (inference.md, "KVCache System"), and split
 * 0 of an empty request, whose output is zero.  Full splits come first in
 * batch order, then each entry's last split, longest first (ties by batch
 * entry), so that the shortest work is dispatched last.
 *   seq_lens    host [batch], KV length of each batch entry
 *   item_batch  host [capacity], written: batch entry of each item
 *   item_index  host [capacity], written: split index of each item
 *   *num_items  the number of items written
 * The decode calls use the list when astr_kv_meta.split_item_batch is set;
 * it must list every split of every entry, as built here (a split left out
 * is neither computed nor merged correctly).
 * Errors: INVAL (null pointer, batch < 0, split_chunk < 1, a negative
 * length, capacity short).
 */
int astr_decode_split_items(const int32_t *seq_lens, int batch, int split_chunk, int32_t *item_batch,
                            int32_t *item_index, int capacity, int *num_items);

/*
 * o[b, h] = sum_j softmax_j(q[b, h] . K_j * sm_scale) V_j over the KV
 * positions j < L_b of request b, L_b = kv_indptr[b+1] - kv_indptr[b], with
 * K_j, V_j = k/v_buffer[layer_id, req_to_token[req_pool_indices[b], j], h / G]
 * (internals.md, "KV Cache Mathematics"; inference.md, "KVCache System":
 * req_to_token is the page table, one slot per token).  sm_scale <= 0 means
 * 1/sqrt(head_dim) (internals.md, "Attention Backend").
 *
 * Split-K: split s of request b covers positions [s*C, min((s+1)*C, L_b)),
 * C = split_chunk.  Pass 1 writes, per (b, h, s < ceil(L_b/C)), the split's
 * normalised output and its natural-log log-sum-exp of scaled scores into
 * o_part / lse_part (the decode_o_part / decode_ml_part buffers of the
 * KVCache record, with the split axis made explicit); pass 2 merges them:
 * M = max_s lse_s, o = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M).
 * When S == 1 the single pass writes `out` directly and o_part / lse_part
 * are not touched (they may then be NULL).
 *   q         device [batch, n_heads, head_dim] act_dtype (already rotated)
 *   o_part    device [batch, n_heads, S, head_dim] float32 scratch
 *   lse_part  device [batch, n_heads, S] float32 scratch (together
 *             astr_decode_workspace_bytes; owned by the caller)
 *   out       device [batch, n_heads, head_dim] act_dtype, written
 *   act_dtype dtype of q and out; must equal m->kv_dtype
 *   m         host; uses the pool fields, req_to_token, num_reqs, max_ctx_len,
 *             req_pool_indices, kv_indptr, batch, max_len (>= every L_b;
 *             it sizes the split axis and, without work items, the grid),
 *             and the decode work items when split_item_batch is set
 *             (then split_item_index, num_split_items >= 1 and
 *             split_item_chunk == split_chunk are required)
 * Requests with L_b == 0 get a zero output.  Errors: INVAL, UNSUPPORTED, LAUNCH.
 */
int astr_decode_attn(const void *q, int n_heads, const astr_kv_meta *m, int layer_id,
                     int split_chunk, float sm_scale, float *o_part, float *lse_part,
                     void *out, astr_dtype act_dtype, void *stream);

/*
 * astr_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with the split-K scratch
 * taken from a device array that the library holds in file scope, one copy
 * per GPU, 160 MiB (ASTR_DECODE_STATIC_SCRATCH_BYTES), placed when the
 * library's code is loaded on that GPU and kept until the process ends.
 * The call itself allocates nothing and frees nothing; the caller passes
 * only q, out and the metadata.  A call whose scratch
 * (astr_decode_workspace_bytes) exceeds the array returns ASTR_E_INVAL
 * before anything is launched.  Every call on one GPU uses that GPU's one
 * array: calls that overlap on one GPU (several streams or threads) race
 * and must be serialised by the caller.  Nothing in the array needs to
 * start at zero: each split's partials are written before the merge reads
 * them.  Arguments and errors as astr_decode_attn.
 */
#define ASTR_DECODE_STATIC_SCRATCH_BYTES ((size_t)160 << 20)
int astr_decode_attn_noalloc(const void *q, int n_heads, const astr_kv_meta *m, int layer_id,
                             int split_chunk, float sm_scale, void *out, astr_dtype act_dtype,
                             void *stream);

/*
 * The decode step with its rotary write fused in (inference.md, "Attention
 * Backend": the paged decode op is handed the step's new k and v and writes
 * them to the cache itself; internals.md, "KV Cache Mathematics": RoPE is
 * applied before the write).  For each request b with L_b >= 1 the new token
 * sits at position L_b - 1 in slot req_to_token[req_pool_indices[b], L_b - 1];
 * this call does, in one launch (plus the merge when S > 1), what
 * astr_rope_kv_write (positions L_b - 1, that slot) followed by
 * astr_decode_attn does, with bit-identical results:
 *   k_buffer[layer, slot] = R(L_b - 1) k_new[b];  v_buffer[layer, slot] = v_new[b]
 *   out[b, h] = attention of R(L_b - 1) q[b, h] over the request's L_b keys
 * q is read only (not rotated in place).
 *   q            device [batch, n_heads, head_dim] bf16, unrotated
 *   k_new, v_new device [batch, m->n_kv_heads, head_dim] bf16, unrotated k
 *   freqs_cis    device [max_pos, head_dim/2, 2] float32, max_pos >= m->max_len
 *   other arguments as astr_decode_attn (act_dtype also covers k_new, v_new).
 * A new-token slot outside the pool is neither written nor attended.
 * Errors: as astr_decode_attn; UNSUPPORTED for a float32 pool; INVAL for null
 * k_new/v_new/freqs_cis or max_pos < max_len.
 */
int astr_decode_attn_write(const void *q, const void *k_new, const void *v_new, int n_heads,
                           const astr_kv_meta *m, int layer_id, const float *freqs_cis, int max_pos,
                           int split_chunk, float sm_scale, float *o_part, float *lse_part,
                           void *out, astr_dtype act_dtype, void *stream);

/* ------------------------------------------------------------------------ */
/* Prefill attention (ragged batch, causal, optional cached prefix)        */
/* ------------------------------------------------------------------------ */

/*
 * Causal attention of each request's new tokens over its whole KV range:
 * request b owns query rows [qo_indptr[b], qo_indptr[b+1]) (e_b of them) and
 * L_b = kv_indptr[b+1] - kv_indptr[b] keys; its first p_b = L_b - e_b
 * positions are a cached prefix (inference.md, "KVCache System": a request
 * resumes after its longest cached page match).  Query i of the request sits
 * at position p_b + i and sees keys j <= p_b + i (internals.md,
 * "Autoregression & Causal Masking", aligned to the end of the KV range).
 * Work is tiled by the query-tile maps q_tile_to_batch / q_tile_to_index:
 * tile t covers rows [q_tile*idx, min(q_tile*(idx+1), e_b)) of request
 * q_tile_to_batch[t] (inference.md, "KVCache System").  Keys and values are
 * read straight from the pool through req_to_token (inference.md, "Attention
 * Backend": ragged prefill addressed by qo_indptr and kv_indptr).
 *   q     device [total_q, n_heads, head_dim] act_dtype (rotated), total_q >=
 *         qo_indptr[batch]; a tile whose rows fall outside [0, total_q) is
 *         skipped (total_q is the row count of q, which the device-side
 *         qo_indptr cannot give the host without a read-back)
 *   out   device, same shape and dtype, written (rows of every tile)
 *   act_dtype  dtype of q and out; must equal m->kv_dtype
 *   m     host; uses the pool fields, req_to_token, num_reqs, max_ctx_len,
 *         req_pool_indices, kv_indptr, qo_indptr, q_tile_to_batch,
 *         q_tile_to_index, batch, max_len, num_q_tiles, q_tile
 *         (q_tile must be 64), and the optional work plan (prefill_units,
 *         num_prefill_units, num_prefill_pairs, prefill_workspace)
 * sm_scale <= 0 means 1/sqrt(head_dim).  A plan changes the order of the
 * softmax sums, not the result beyond rounding.  Errors: INVAL (also: split
 * tiles without a workspace, more split tiles than half the units, a
 * workspace smaller than its plan needs, units not 16-byte aligned, more
 * units than 16 * num_q_tiles), UNSUPPORTED, LAUNCH.
 */
int astr_prefill_attn(const void *q, int total_q, int n_heads, const astr_kv_meta *m,
                      int layer_id, float sm_scale, void *out, astr_dtype act_dtype, void *stream);

/*
 * Workspace of a prefill work plan with `pairs` split tiles: per pair, KV
 * head and group of 4 query heads, a completion count (int32) and the two
 * units' partial results (the float32 O accumulators and, per row, the
 * running max and the row sum).  The counts must be zero before the first
 * call that uses the workspace; every call leaves them zero again.  Calls
 * that share a workspace must not run concurrently.  The layout is that of
 * the head_dim-128 kernel, the only one that follows plans.  0 for no pairs
 * and on bad input.
 */
size_t astr_prefill_workspace_bytes(int pairs, int n_heads, int head_dim);

/*
 * The prefill work plan of a step (host only).  Its reading of the pages:
 * the pages tile prefill work by query tiles (inference.md, "KVCache
 * System") and leave open how tiles are scheduled.  With one workgroup per
 * compute unit, a batch whose longest tiles carry much more than the mean
 * load finishes when its longest tile does; splitting such a tile's keys in
 * two halves shortens that critical path.  The halves merge as the decode
 * splits do (inference.md, "KVCache System": split-K partial outputs kept
 * with their partial max and sum, from which the softmax over the union of
 * the key sets follows exactly).
 * Rule: tile t sees n_t = ceil(kv_end_t / 32) key steps, kv_end_t = p_b +
 * row0 + rows (0 steps for a tile with inconsistent metadata).  Costs, in
 * steps of 32 keys (measured on MI355X: ~1 us per step, ~5 us of prologue,
 * ~2 us to store a tile's output, ~3 us to publish a half's state, ~3 us to
 * merge): a whole tile 7 + n_t (0.1 when skipped), a lower half [0, h) 8.5
 * + h, an upper half [h, end) 9.5 + n_t - h.  Candidates: no split; the
 * tiles with n_t > floor(max_t n_t * k / 10), k = 9 .. 3, cut at h =
 * n_t / 2; the N longest tiles (ties: tile order), N in {1, 2, 3, 4, 5, 6,
 * 8, 10, 12, 16} below num_q_tiles, cut at h = max(1, floor(3 n_t / 10))
 * (only tiles with n_t >= 2 are cut).  For each, the units are listed by decreasing cost (ties: tile
 * order, then lower half first) and dealt to the 8 XCDs in that order,
 * each to an XCD where it would end first; among those, an XCD that already
 * holds one to three units of the same batch entry comes first, then fewer
 * units queued, then the lower XCD.  A request's tiles all read its
 * page-aligned key/value prefix (inference.md, "KVCache System") and each
 * XCD has its own L2, so tiles kept together fetch the prefix fewer times;
 * at most four per XCD, as more tiles of one request running side by side
 * on one XCD measured slower.  An XCD runs its queue in order on num_cus / 8 compute units,
 * one workgroup per compute unit, the unit's workgroups_per_tile workgroups
 * on the ones free first.  The candidate with the earliest simulated end
 * (the first listed on ties) wins if it ends at least 10% before the
 * unsplit list.  Entry 8k + x of the
 * plan is the k-th unit of XCD x (the kernel runs unit u on XCD u % 8);
 * shorter queues are padded with units of tile -1 and 0 rows, which do
 * nothing.
 * A unit also carries its tile's request row req_pool_indices[b], first
 * query row qo_indptr[b] + row0, rows and first row's position p_b + row0,
 * so that the kernel reads one descriptor instead of the tile maps.
 *   qo_indptr, kv_indptr  host [batch + 1]; req_pool_indices host [batch];
 *   q_tile_to_batch, q_tile_to_index host [num_q_tiles]; q_tile rows per
 *   tile (64); workgroups_per_tile = n_heads / 4 for the kernel that follows
 *   plans; num_cus >= 8
 *   units       host [capacity][8], written (layout of astr_kv_meta.prefill_units)
 *   *num_units, *num_pairs  written
 * capacity >= 16 * num_q_tiles always suffices.
 * Errors: INVAL (null pointer, negative size, num_cus < 8, capacity short).
 */
int astr_prefill_plan(const int32_t *qo_indptr, const int32_t *kv_indptr, const int32_t *req_pool_indices,
                      int batch, const int32_t *q_tile_to_batch, const int32_t *q_tile_to_index,
                      int num_q_tiles, int q_tile, int workgroups_per_tile, int num_cus, int32_t *units,
                      int capacity, int *num_units, int *num_pairs);

/* ------------------------------------------------------------------------ */
/* Page-table builder (host only; no device calls)                          */
/* ------------------------------------------------------------------------ */

/*
 * PagePool (inference.md, "KVCache System"; internals.md, "Cache
 * Architecture").  mode 0 = contiguous: slot = req_idx * max_ctx_len + pos,
 * no dynamic allocation (needs pool_slots >= max_reqs * max_ctx_len).
 * mode 1 = paged: pages of page_size slots taken from a bitmask allocator
 * with reference counts; with page_size > 1 a radix cache of complete,
 * materialised token pages lets a new request reuse an exact page-aligned
 * prefix (token tuples compared exactly under the same parent page).
 *
 * Allocation order (fixed so that tables are reproducible): the lowest free
 * request slot and the lowest free logical page are taken first; logical
 * page p maps to physical page page_perm[p] (identity when page_perm is NULL);
 * slot = physical_page * page_size + pos % page_size.  Unused table entries
 * hold -1.  A handle is single-threaded and owns host memory only.
 */
typedef struct astr_pagepool astr_pagepool;

/* page_perm: host [pool_slots / page_size] permutation, copied; may be NULL.
 * Errors: INVAL (bad sizes or page_perm not a permutation), NOMEM (host allocation). */
int astr_pagepool_create(astr_pagepool **out, int mode, int64_t pool_slots, int page_size,
                         int max_reqs, int max_ctx_len, const int32_t *page_perm);
void astr_pagepool_destroy(astr_pagepool *pp);

/* Take the lowest free request slot.  With radix sharing on and tokens given
 * (host [n_tokens]), reuse the longest chain of cached complete pages that
 * matches tokens[0 : page_size*k], k <= (n_tokens - 1) / page_size (at least
 * one token is left to compute); *cached_len = page_size * k is then the
 * request's length.  Errors: INVAL, NOMEM (no free request slot). */
int astr_pagepool_admit(astr_pagepool *pp, const int32_t *tokens, int n_tokens,
                        int *req_idx, int *cached_len);

/* Give request req_idx slots for positions [len, len + n_new), evicting
 * least recently used cached pages first when the free pages are short (see
 * astr_pagepool_evict).  Errors: INVAL (not live, or length > max_ctx_len),
 * NOMEM (free plus evictable pages are short; nothing changes). */
int astr_pagepool_extend(astr_pagepool *pp, int req_idx, int n_new);

/* Per-step metadata for batch entries b < batch (request req_idx[b], q_lens[b]
 * new tokens at its last q_lens[b] positions), into caller-owned host arrays:
 *   seq_lens[batch], out_cache_loc[sum q_lens] (qo order), kv_indptr[batch+1],
 *   qo_indptr[batch+1], q_tile_to_batch / q_tile_to_index [tile_capacity]
 *   (tiles of q_tile rows listed heaviest first: by decreasing KV extent
 *   seen by the tile's last row, ties by batch entry then tile index; may be
 *   NULL when tile_capacity is 0), *num_q_tiles, *max_len.
 * Errors: INVAL (request not live, q_len > seq_len, tile capacity short). */
int astr_pagepool_bind(astr_pagepool *pp, const int32_t *req_idx, const int32_t *q_lens,
                       int batch, int q_tile, int32_t *seq_lens, int32_t *out_cache_loc,
                       int32_t *kv_indptr, int32_t *qo_indptr, int32_t *q_tile_to_batch,
                       int32_t *q_tile_to_index, int tile_capacity, int *num_q_tiles,
                       int *max_len);

/* Record the complete pages among the request's first n_materialized
 * positions (tokens host [n_materialized]) in the radix; partial pages stay
 * private.  A page already cached under the same parent and tokens is kept
 * and the request's copy stays private.  No-op without radix sharing. */
int astr_pagepool_insert(astr_pagepool *pp, int req_idx, const int32_t *tokens,
                         int n_materialized);

/* Drop the request's page references (pages reaching zero are freed) and
 * free its request slot; its table row returns to -1. */
int astr_pagepool_release(astr_pagepool *pp, int req_idx);

/* A finished request (inference.md, "KVCache System": what completion
 * records).  tokens host [n_tokens] is its prompt plus every generated token;
 * the last one was sampled but never passed through the model, so only the
 * first n_tokens - 1 have KV: the complete pages among those are cached as by
 * astr_pagepool_insert, then the request is released (its partial page and
 * every page no one else holds return to the free set).
 * Errors: INVAL (not live, tokens NULL with n_tokens > 0). */
int astr_pagepool_complete(astr_pagepool *pp, int req_idx, const int32_t *tokens, int n_tokens);

/* LRU eviction (same section: the allocator's ref-counted pages with LRU
 * eviction).  A cached page is evictable when only the radix holds it and it
 * has no cached children; the least recently used goes first, where each
 * admit or insert call is one tick and uses every cached page it matches or
 * passes over.  astr_pagepool_extend evicts by itself when the free pages are
 * short, just enough of them, and evicts nothing when even all evictable
 * pages would not be enough (NOMEM).  This call frees up to n_pages cached
 * pages ahead of need and returns how many it freed (0 without radix
 * sharing; -1 and INVAL on a bad argument). */
int64_t astr_pagepool_evict(astr_pagepool *pp, int64_t n_pages);

/* Introspection: pages held by the radix; pages evicted since creation. */
int64_t astr_pagepool_cached_pages(const astr_pagepool *pp);
int64_t astr_pagepool_evicted_pages(const astr_pagepool *pp);

/* The host table [max_reqs, max_ctx_len] int32 owned by the handle, valid
 * until the next call that changes it or destroy (NULL on bad handle). */
const int32_t *astr_pagepool_table(const astr_pagepool *pp);

/* Introspection: free pages, reference count of a logical page (-1 if out of range). */
int64_t astr_pagepool_free_pages(const astr_pagepool *pp);
int astr_pagepool_page_ref(const astr_pagepool *pp, int64_t logical_page);

#ifdef __cplusplus
}
#endif

#endif /* ASTR_H */
