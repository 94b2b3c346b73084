// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// ---------------------------------------------------------------- KV append
struct KvWriteArgs {
    const void *k;
    const void *v;
    void *k_cache;
    void *v_cache;
    const int64_t *slot_mapping;
    int64_t num_tokens;
    int64_t k_token_stride;  // elements
    int64_t v_token_stride;  // elements
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t elem_bytes;
};

hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- decode
// Work split chosen on the host from sizes only (no device reads).
struct DecodePlan {
    int32_t part_tokens;  // tokens per partition (multiple of 16)
    int32_t max_parts;    // partitions of the longest possible sequence
    int32_t waves;        // waves per workgroup
    size_t workspace_bytes;
    size_t ws_acc_offset;  // bytes from the workspace start
    size_t ws_ml_offset;
};

struct DecodeArgs {
    void *out;
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    float *ws_acc;  // [num_seqs][num_q_heads][max_parts][head_dim]   un-normalised
    float *ws_ml;   // [num_seqs][num_q_heads][max_parts][2]          (max, exp-sum)
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int32_t part_tokens;
    int32_t max_parts;
    float scale_log2;  // scale * log2(e): scores are kept in base-2 exponent units
};

constexpr int kSubTile = 16;      // tokens scored together by one wave
constexpr int kMaxParts = 4096;   // reduce kernel keeps one weight per partition in LDS

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                       int32_t max_context_len);

bool decode_supported(int32_t dtype, int32_t head_dim, int32_t group);

// Launches the partition kernel and, when any sequence can span several
// partitions, the merge kernel.  dtype: 0 f32, 1 f16, 2 bf16.
hipError_t launch_attn_decode(int32_t dtype, int32_t head_dim, int32_t group,
                              const DecodeArgs &a, const DecodePlan &plan,
                              hipStream_t stream);

}  // namespace pkv
