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
    if (slot < 0 || slot >= a.num_slots) return;   // skipped, or outside the pool
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

// Input checks (a debugging aid): the device-resident data the decode and
// append calls take on trust.  One thread per sequence checks its length and
// the table entries it uses; one thread per token checks its slot, and marks
// it in a bitmap to find repeats.  Every violation is counted; one of them is
// described.
__device__ void report(int64_t *result, int kind, int64_t index, int64_t value) {
    auto *r = reinterpret_cast<unsigned long long *>(result);
    atomicAdd(r, 1ull);
    if (atomicCAS(r + 1, 0ull, (unsigned long long)kind) == 0ull) {
        result[2] = index;
        result[3] = value;
    }
}

__global__ __launch_bounds__(256) void check_init_kernel(CheckArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx == 0) {
        a.result[0] = 0;
        a.result[1] = 0;
        a.result[2] = -1;
        a.result[3] = 0;
    }
    for (int64_t w = idx; w < a.bitmap_words; w += (int64_t)gridDim.x * blockDim.x) a.bitmap[w] = 0u;
}

__global__ __launch_bounds__(256) void check_kernel(CheckArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx < a.num_seqs) {
        const int L = a.context_lens[idx];
        if (L < 0 || L > a.max_context_len) {
            report(a.result, 1, idx, L);
        } else {
            const int n = (L + a.block_size - 1) / a.block_size;
            for (int j = 0; j < n; ++j) {
                const int32_t b = a.block_tables[idx * a.max_blocks_per_seq + j];
                if (b < 0 || b >= a.num_blocks) {
                    report(a.result, 2, idx, b);
                    break;
                }
            }
        }
    }
    if (a.slot_mapping != nullptr && idx < a.num_tokens) {
        const int64_t s = a.slot_mapping[idx];
        if (s >= 0) {
            if (s >= a.num_blocks * (int64_t)a.block_size) {
                report(a.result, 3, idx, s);
            } else if (a.bitmap != nullptr) {
                const uint32_t bit = 1u << (s & 31);
                if (atomicOr(a.bitmap + (s >> 5), bit) & bit) report(a.result, 4, idx, s);
            }
        }
    }
}

}  // namespace

hipError_t launch_check(const CheckArgs &a, hipStream_t stream) {
    const int64_t words = a.bitmap ? a.bitmap_words : 0;
    int64_t init_groups = (words + 255) / 256;
    init_groups = init_groups < 1 ? 1 : (init_groups > 4096 ? 4096 : init_groups);
    check_init_kernel<<<dim3((unsigned)init_groups), dim3(256), 0, stream>>>(a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    const int64_t n = a.num_seqs > a.num_tokens ? a.num_seqs : a.num_tokens;
    const int64_t groups = n > 0 ? (n + 255) / 256 : 1;
    check_kernel<<<dim3((unsigned)groups), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

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
