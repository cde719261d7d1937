// Host-side launchers of the HIP kernels (one translation unit per kernel
// family).  Arguments have been validated by the C entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace astr {

struct PoolView {
    void *k_layer;          // k_buffer + layer_id * pool_slots * n_kv_heads * head_dim
    void *v_layer;
    int64_t pool_slots;
    int n_kv_heads;
    int head_dim;
    int dtype;              // astr_dtype
};

struct RopeArgs {
    void *q;
    const void *k;
    const void *v;
    const int32_t *positions;
    const int32_t *out_cache_loc;
    int n_tokens;
    int n_heads;
    const float *freqs;
    int max_pos;
    PoolView pool;
};

struct DecodeArgs {
    const void *q;
    void *out;
    float *o_part;
    float *lse_part;
    PoolView pool;
    const int32_t *req_to_token;
    int num_reqs;
    int max_ctx_len;
    const int32_t *req_pool_indices;
    const int32_t *kv_indptr;
    int batch;
    int n_heads;
    int split_chunk;
    int n_splits;
    float scale_log2;       // sm_scale * log2(e)
    // work items (batch entry, split); num_items == 0: one slot per (entry, split)
    const int32_t *item_batch;
    const int32_t *item_index;
    int num_items;
    // fused rotary write of the step's new token (null k_new: plain decode)
    const void *k_new;
    const void *v_new;
    const float *freqs;
    int max_pos;
};

struct PrefillArgs {
    const void *q;
    void *out;
    int total_q;            // rows of q and out
    PoolView pool;
    const int32_t *req_to_token;
    int num_reqs;
    int max_ctx_len;
    const int32_t *req_pool_indices;
    const int32_t *qo_indptr;
    const int32_t *kv_indptr;
    const int32_t *q_tile_to_batch;
    const int32_t *q_tile_to_index;
    int batch;
    int num_q_tiles;
    int q_tile;
    int n_heads;
    float scale_log2;
    // work plan (num_units 0: one unit per tile); part_cnt / part: workspace
    const int32_t *units;
    int num_units;
    int num_pairs;
    int32_t *part_cnt;
    float *part;
};

// Prefill workspace of a plan: per (pair, KV head, group of 4 query heads) a
// completion count, then two partial results of kPrefillPartFloats floats:
// O^T accumulators [4 row blocks][4 heads][8 column blocks][64 lanes][4] and
// (max, sum) [4 row blocks][4 heads][2][64 lanes] (one 16-byte store per lane,
// a wave's covering 1 KB).
constexpr int64_t kPrefillPartFloats = 4 * 4 * 8 * 64 * 4 + 4 * 4 * 2 * 64;
inline int64_t prefill_part_slots(int64_t pairs, int n_heads) { return pairs * ((n_heads + 3) / 4); }
inline int64_t prefill_counts_bytes(int64_t slots) { return (4 * slots + 255) / 256 * 256; }

// Largest byte stride of a structured-buffer record (14-bit field); the bf16
// prefill addresses the pool as records of this size or less.
constexpr int64_t kMaxRecordStride = 16383;

hipError_t launch_rope_table(float *freqs, int max_pos, int head_dim, double theta, hipStream_t s);
hipError_t launch_rope_kv_write(const RopeArgs &a, hipStream_t s);
hipError_t launch_rope_backward(void *grad, const int32_t *positions, int n_tokens, int n_heads, int head_dim,
                                int dtype, const float *freqs, int max_pos, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
// Capacity of the file-scope split-K scratch of the allocation-free decode,
// and its address on the current device (looked up once per device).
constexpr size_t kStaticDecodeScratchBytes = size_t(160) << 20;
hipError_t static_decode_scratch(float **ptr);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);
hipError_t launch_ceiling_stream_read(const void *buf, uint64_t bytes, int workgroups, bool nontemporal,
                                      uint32_t *sink, hipStream_t s);
hipError_t launch_ceiling_mfma_loop(int workgroups, int iters, float *sink, hipStream_t s);

}  // namespace astr
