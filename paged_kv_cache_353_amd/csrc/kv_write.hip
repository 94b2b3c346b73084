// KV append: copy each new token's K/V rows into its slot of the paged cache;
// and the block copy that copy-on-write needs.
//
// "PagedAttention核心思想" section 2.4.2: a generated token is stored in the
// next free slot of its sequence's last block (a new block is taken only when
// that one is full); the slot is physical_block * block_size + offset.
//
// One thread moves one 16-byte chunk of K and the matching chunk of V.  Rows
// of a (token, head) are head_dim * elem_bytes contiguous bytes on both sides,
// so consecutive threads read and write consecutive 16-byte chunks.  The copy
// is a bit copy: no conversion, NaN payloads and signed zeros survive.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs a, int chunks_per_row) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_token = (int64_t)a.num_kv_heads * chunks_per_row;
    if (idx >= a.num_tokens * per_token) return;
    const int64_t n = idx / per_token;
    const int32_t rem = (int32_t)(idx - n * per_token);
    const int32_t h = rem / chunks_per_row;
    const int32_t c = rem - h * chunks_per_row;
    const int64_t slot = a.slot_mapping[n];
    if (slot < 0) return;
    const int64_t blk = slot / a.block_size;
    const int64_t off = slot - blk * a.block_size;
    const int64_t row_bytes = (int64_t)a.head_dim * a.elem_bytes;
    const int64_t dst = ((blk * a.num_kv_heads + h) * a.block_size + off) * row_bytes + (int64_t)c * 16;
    const int64_t src_k = n * a.k_token_stride * a.elem_bytes + h * row_bytes + (int64_t)c * 16;
    const int64_t src_v = n * a.v_token_stride * a.elem_bytes + h * row_bytes + (int64_t)c * 16;
    const u32x4 kx = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.k) + src_k);
    const u32x4 vx = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.v) + src_v);
    *reinterpret_cast<u32x4 *>(static_cast<char *>(a.k_cache) + dst) = kx;
    *reinterpret_cast<u32x4 *>(static_cast<char *>(a.v_cache) + dst) = vx;
}

// Block copy (copy-on-write): one workgroup per (src, dst) pair moves the
// whole block, every KV head and row, of K and of V, 16 bytes per thread per
// step.  A block is contiguous in both caches, so reads and writes coalesce.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
    const int64_t pair = blockIdx.x;
    const int64_t src = a.pairs[2 * pair];
    const int64_t dst = a.pairs[2 * pair + 1];
    if (src < 0 || dst < 0) return;
    const int64_t chunks = a.block_bytes / 16;
    const char *ks = static_cast<const char *>(a.k_cache) + src * a.block_bytes;
    const char *vs = static_cast<const char *>(a.v_cache) + src * a.block_bytes;
    char *kd = static_cast<char *>(a.k_cache) + dst * a.block_bytes;
    char *vd = static_cast<char *>(a.v_cache) + dst * a.block_bytes;
    for (int64_t i = threadIdx.x; i < chunks; i += blockDim.x) {
        const u32x4 kx = *reinterpret_cast<const u32x4 *>(ks + i * 16);
        const u32x4 vx = *reinterpret_cast<const u32x4 *>(vs + i * 16);
        *reinterpret_cast<u32x4 *>(kd + i * 16) = kx;
        *reinterpret_cast<u32x4 *>(vd + i * 16) = vx;
    }
}

// Append at the end of each context: the token of sequence i goes to
// position L_i - 1 (L_i = context_lens[i], clamped to max_context_len), whose
// slot comes from the sequence's Block Table.  One workgroup per sequence;
// sequences with L_i == 0 write nothing.
__global__ __launch_bounds__(256) void append_last_kernel(AppendLastArgs a) {
    const int i = blockIdx.x;
    int L = a.context_lens[i];
    L = L < a.max_context_len ? L : a.max_context_len;
    if (L <= 0) return;
    const int pos = L - 1;
    const int j = pos / a.block_size;
    const int64_t phys = a.block_tables[(int64_t)i * a.max_blocks_per_seq + j];
    const int64_t row_bytes = (int64_t)a.head_dim * a.elem_bytes;
    const int chunks = (int)(row_bytes / 16);
    for (int idx = threadIdx.x; idx < a.num_kv_heads * chunks; idx += blockDim.x) {
        const int h = idx / chunks, c = idx - h * chunks;
        const int64_t src = ((int64_t)i * a.num_kv_heads + h) * row_bytes + (int64_t)c * 16;
        const int64_t dst = ((phys * a.num_kv_heads + h) * a.block_size + (pos - j * a.block_size)) * row_bytes +
                            (int64_t)c * 16;
        const u32x4 kx = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.k_new) + src);
        const u32x4 vx = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.v_new) + src);
        *reinterpret_cast<u32x4 *>(static_cast<char *>(a.k_cache) + dst) = kx;
        *reinterpret_cast<u32x4 *>(static_cast<char *>(a.v_cache) + dst) = vx;
    }
}

}  // namespace

hipError_t launch_append_last(const AppendLastArgs &a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    append_last_kernel<<<dim3((unsigned)a.num_seqs), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyBlocksArgs &a, hipStream_t stream) {
    if (a.num_pairs == 0) return hipSuccess;
    copy_blocks_kernel<<<dim3((unsigned)a.num_pairs), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t stream) {
    const int chunks_per_row = a.head_dim * a.elem_bytes / 16;
    const int64_t total = a.num_tokens * a.num_kv_heads * chunks_per_row;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    kv_write_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a, chunks_per_row);
    return hipGetLastError();
}

}  // namespace pkv
