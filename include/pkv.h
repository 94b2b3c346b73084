/*
 * pkv.h -- C ABI of libpkv.so: paged-KV-cache decode attention for MI355X (gfx950).
 *
 * The KV cache of every sequence is split into fixed-size physical blocks that
 * may sit anywhere in one pool; a per-sequence Block Table maps logical block j
 * to its physical block id ("PagedAttention核心思想", sections 2.2-2.3; CSDN
 * answer "VLLM中PagedAttention如何降低显存碎片？", section 三 items 1-4).
 *
 * Layouts (row-major, element counts):
 *   k_cache, v_cache  [num_blocks, num_kv_heads, block_size, head_dim]
 *                     one block holds block_size tokens for every KV head
 *                     ("PagedAttention核心思想" section 2.3)
 *   block_tables      int32 [num_seqs, max_blocks_per_seq]; entry [i][j] is the
 *                     physical block holding tokens [j*block_size, (j+1)*block_size)
 *                     of sequence i.  Entries j >= ceil(context_lens[i]/block_size)
 *                     are never read.
 *   context_lens      int32 [num_seqs]; tokens attended by sequence i
 *   q, out            [num_seqs, num_q_heads, head_dim], contiguous
 *   k, v (new tokens) [num_tokens, num_kv_heads, head_dim]; tokens may be strided
 *   slot_mapping      int64 [num_tokens]; slot = physical_block*block_size + offset
 *
 * Ownership: every pointer argument is device memory owned by the caller.  The
 * library allocates nothing and is reentrant; its global state is caches filled
 * on first use (kernel occupancy per configuration, compute units per device)
 * and the per-device static array behind paged_decode_step_static.  All
 * work is queued asynchronously on `stream` (NULL = the null stream).  Outputs
 * are `out` and the caches; `out` must not alias q or the caches, and k/v must
 * not alias the caches.
 *
 * Errors: every call returns a pkv_status_t.  Arguments are checked on the host
 * only (no device reads, no synchronisation); a failed check returns before
 * anything is launched.  Preconditions on device-resident data are NOT checked
 * by the compute calls (paged_check_inputs checks them on request): block ids
 * used by a sequence lie in [0, num_blocks); non-negative slots are distinct;
 * 0 <= context_lens[i] <= max_context_len.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, out, k, v and the caches. */
typedef enum pkv_dtype {
    PKV_F32 = 0,
    PKV_F16 = 1,
    PKV_BF16 = 2
} pkv_dtype_t;

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_NULL = 1,        /* a required pointer is NULL                        */
    PKV_ERR_SHAPE = 2,       /* a size is out of range or sizes disagree          */
    PKV_ERR_DTYPE = 3,       /* unknown dtype code                                */
    PKV_ERR_UNSUPPORTED = 4, /* valid, but no kernel is built for it (head_dim,   */
                             /* block size or query-per-KV-head group)            */
    PKV_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required        */
    PKV_ERR_ALIGN = 6,       /* a pointer or token stride is not 16-byte aligned  */
    PKV_ERR_HIP = 7          /* the HIP runtime reported an error at launch       */
} pkv_status_t;

/* Static text for a status code (never NULL). */
const char *pkv_status_string(int status);

/* Library ABI version (major*10000 + minor*100 + patch). */
int pkv_version(void);

/*
 * paged_kv_write -- append new tokens' K/V to the paged cache.
 *
 * For every token n with slot s = slot_mapping[n] >= 0 and every KV head h:
 *   k_cache[s / block_size, h, s % block_size, :] = k[n, h, :]   (bit copy)
 *   v_cache[s / block_size, h, s % block_size, :] = v[n, h, :]
 * A negative slot skips the token, and so does a slot at or past
 * num_blocks*block_size (the kernel checks the bound).  Defined by "PagedAttention核心思想" section
 * 2.4.2 (a new token goes into the next slot of the last block; a fresh block
 * is taken only when the last one is full) and the CSDN answer's flow chart in
 * section 四 (append a page, update the mapping).
 *
 *   k, v             new tokens, element (n, h, d) at n*token_stride + h*head_dim + d
 *   k_token_stride,
 *   v_token_stride   elements between consecutive tokens (>= num_kv_heads*head_dim)
 *   num_tokens       may be 0 (nothing is launched)
 *   head_dim         64 or 128;  block_size > 0;  num_blocks > 0
 * Pointers and strides in bytes must be multiples of 16.
 */
int paged_kv_write(const void *k, const void *v, void *k_cache, void *v_cache,
                   const int64_t *slot_mapping, int64_t num_tokens,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int64_t num_blocks, int64_t k_token_stride, int64_t v_token_stride,
                   int32_t dtype, hipStream_t stream);

/*
 * paged_copy_blocks -- copy whole physical blocks (copy-on-write).
 *
 * For every pair n with src = block_pairs[2n] >= 0 and dst = block_pairs[2n+1]
 * >= 0, block dst of both caches becomes a bit copy of block src: every KV
 * head and every row.  Shared blocks are read-only; a write into a block whose
 * reference count is above one first copies it to a fresh block
 * ("PagedAttention核心思想" section 2.4.3; "PagedAttention技术解析" section
 * 2.1 on reference counts).  Copying the whole block leaves the valid rows
 * identical; rows past a sequence's end are never read.
 *
 *   block_pairs   int64 [num_pairs][2] on the device; a negative entry skips
 *                 the pair
 * Preconditions (not checked, device data): ids below num_blocks; no block is
 * the destination of two pairs, or both a source and a destination.
 */
int paged_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_pairs,
                      int64_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int64_t num_blocks, int32_t dtype,
                      hipStream_t stream);

/*
 * Bytes of device workspace paged_attn_decode needs for these sizes (0 for
 * invalid sizes; the decode call reports those).  The work of a batch is cut
 * into equal pieces, one per wave the GPU runs at once; a (sequence, KV head)
 * pair whose context is split between waves leaves one partial result per
 * piece here (running max, exp-sum and un-normalised output, fp32), merged by
 * the last wave to finish, which it finds through arrival counters (one per
 * pair, one per group of pieces).  The counters occupy the first
 * PKV_DECODE_COUNTER_BYTES bytes of every workspace, whatever the sizes (so
 * num_seqs * num_kv_heads <= 2^20); partial results follow.  The size depends
 * on num_seqs, num_kv_heads, the group size and head_dim; block_size and
 * max_context_len are accepted for symmetry with the decode call.
 */
/* Bytes at the start of every decode workspace that hold arrival counters:
 * (2^20 + 8192 + 2^20) int32. */
#define PKV_DECODE_COUNTER_BYTES ((size_t)8421376)

size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_context_len);

/*
 * paged_attn_decode -- one query token per sequence attends over its paged KV cache.
 *
 * For sequence i and query head h (KV head g = h / (num_q_heads/num_kv_heads)):
 *   s_t = scale * dot(q[i,h,:], K_t)      t in [0, context_lens[i])
 *   out[i,h,:] = sum_t softmax(s)_t * V_t
 * where K_t, V_t are row t % block_size of KV head g in physical block
 * block_tables[i][t / block_size].  The table is walked inside the kernel,
 * block by block, with a numerically stable (running-max) softmax
 * ("PagedAttention核心思想" section 2.5; "PagedAttention技术解析" sections 2.2
 * and 3.1; CSDN answer section 三 items 4-6 and 9, and section 四 on the
 * partitioned second version).  Slots past context_lens[i] in the last block
 * are never used.  context_lens[i] == 0 gives out[i] = 0.  Accumulation is
 * fp32; out is rounded once to its dtype (round to nearest even).
 *
 *   num_q_heads % num_kv_heads == 0 and the group size is 1, 2, 4 or 8
 *   head_dim 64 or 128; block_size a multiple of 16 up to 256
 *   max_blocks_per_seq*block_size >= max_context_len
 *   num_seqs * num_kv_heads <= 2^20 and
 *   num_seqs * num_kv_heads * ceil(max_context_len / 16) < 2^31
 *   workspace: >= paged_attn_decode_workspace_size(...) bytes of device memory,
 *              256-byte aligned, whose first PKV_DECODE_COUNTER_BYTES bytes are
 *              zero-filled once before its first use.  Every call returns them
 *              to zero (the rest needs no initialisation), so one workspace
 *              serves any number of later calls, of any shape it is large
 *              enough for, on the same stream; calls that may run at the same
 *              time need separate workspaces.
 * Results depend only on the logical contents and the sizes (and on the GPU's
 * compute-unit count, which fixes how work is split): they are bitwise
 * reproducible and do not change when blocks are relabelled or resized.
 */
int paged_attn_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                      int64_t num_blocks, int32_t max_context_len, float scale,
                      int32_t dtype, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * paged_decode_step -- one decode step in one launch: append each sequence's
 * new token to the cache and attend over the context including it.
 *
 * For every sequence i with L = context_lens[i] >= 1, the new token sits at
 * position L - 1: its K/V (k_new[i], v_new[i]) are written to that position's
 * slot, block_tables[i][(L-1) / block_size] * block_size + (L-1) % block_size
 * (a token goes into the next slot of the last block, "PagedAttention核心思想"
 * section 2.4.2), and
 *   out[i,h,:] = sum_t softmax(s)_t * V_t,  t in [0, L),
 * exactly as paged_kv_write followed by paged_attn_decode would give, with the
 * new token's K/V taken from k_new/v_new (so nothing reads the slot while it
 * is being written).  L == 0 gives out[i] = 0 and writes nothing.
 *
 *   k_new, v_new   [num_seqs, num_kv_heads, head_dim], contiguous, 16-byte
 *                  aligned, same dtype as the caches
 *   other arguments, preconditions and the workspace as for paged_attn_decode;
 *   in addition, block_tables[i] holds the block of position L - 1.
 */
int paged_decode_step(void *out, const void *q, const void *k_new, const void *v_new,
                      void *k_cache, void *v_cache, const int32_t *block_tables,
                      const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                      float scale, int32_t dtype, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * paged_decode_step_static -- paged_decode_step for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops and harnesses
 * that forbid hipMalloc.  It takes no workspace and calls no allocator; its
 * arrival counters and partial results live in a fixed device array of
 * 24 MiB per GPU that the library holds until the process ends.  The first
 * call on a device (with that device current, not under stream capture)
 * looks the array up and clears its counters on the given stream; every call
 * leaves them zero.  Every call on one GPU shares that array: calls that may
 * overlap on one GPU (two streams, two threads) race and give wrong results.
 *
 * Arguments, preconditions and results are those of paged_decode_step (both
 * run the same kernel and give bitwise equal outputs and caches), with these
 * limits:
 *   num_seqs * num_kv_heads <= 16384, and the partial results of that many
 *   units plus one per wave of the grid fit the array
 *   (about (1024 + units) * group * head_dim * 8 bytes)  -> PKV_ERR_WORKSPACE
 *   configurations that paged_decode_step serves with its many-column kernel
 *   (group sizes other than 1, 2, 4, 8, and any whose one-query kernel
 *   would spill registers: none at present)
 *                                                       -> PKV_ERR_UNSUPPORTED
 *   first call on a device under stream capture         -> PKV_ERR_HIP
 */
int paged_decode_step_static(void *out, const void *q, const void *k_new, const void *v_new,
                             void *k_cache, void *v_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                             float scale, int32_t dtype, hipStream_t stream);

/*
 * paged_attn_decode_multi -- several query tokens per sequence.
 *
 * Parallel sampling, beam search and the verification of drafted tokens give
 * a sequence more than one query in a step ("PagedAttention核心思想" section
 * 2.4.3).  The T = num_query_tokens new tokens of sequence i are its last T
 * positions, already written to the cache (paged_kv_write), and each attends
 * to every position up to and including its own:
 *   out[i,j,h,:] = sum_t softmax(s)_t * V_t,  t in [0, L_i - T + j + 1),
 * with s as for paged_attn_decode; a query whose window is empty (L_i < T - j)
 * gets zeros.  The cache is read block by block through the table exactly as
 * for one query ("PagedAttention核心思想" section 2.5).
 *
 *   out, q        [num_seqs, num_query_tokens, num_q_heads, head_dim], 16-byte
 *                 aligned, dtype of the caches
 *   dtype         PKV_F32, PKV_F16 or PKV_BF16; products run on matrix cores
 *                 with fp32 accumulation; the softmax weights multiply V as
 *                 fp32, as fp16 (11 significant bits) or as a bf16 head plus a
 *                 bf16 remainder (about 16 bits)
 *   head_dim      64 or 128; block_size a power of two from 16 to 256; any
 *                 num_q_heads / num_kv_heads
 *   workspace     >= paged_attn_decode_multi_workspace_size(...) bytes,
 *                 256-byte aligned, first PKV_DECODE_COUNTER_BYTES zero once
 *                 (every call leaves them zero; same contract as
 *                 paged_attn_decode)
 * Other arguments, preconditions and errors as for paged_attn_decode.
 */
size_t paged_attn_decode_multi_workspace_size(int32_t num_seqs, int32_t num_query_tokens,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim);
int paged_attn_decode_multi(void *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            int32_t num_seqs, int32_t num_query_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t max_blocks_per_seq, int64_t num_blocks,
                            int32_t max_context_len, float scale, int32_t dtype,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attn_decode_shared -- one query per sequence, with the shared prefix
 * of forked sequences read once for the whole group.
 *
 * Forks of one request (parallel sampling, beam search) point their Block
 * Tables at the same physical blocks for the prompt they share
 * ("PagedAttention核心思想" section 2.4.3; "PagedAttention技术解析" section 2.1).
 * The result is exactly paged_attn_decode's; the sharing only changes how
 * often those blocks are read: the prefix of every group is streamed once for
 * all query heads of all its members, each member then streams its own
 * suffix, and the two partial softmax results are merged.
 *
 *   group_starts  int32 [num_groups + 1] on the device: the members of group g
 *                 are sequences group_starts[g] .. group_starts[g+1] - 1
 *                 (consecutive; group_starts[0] = 0, group_starts[num_groups]
 *                 = num_seqs, non-decreasing)
 *   prefix_lens   int32 [num_seqs] on the device: P_i, the leading positions
 *                 sequence i shares with its group (0 for none)
 * Preconditions (device data, not checked): within a group P_i is the same,
 * P_i <= L_i, and block_tables[i][j] is the same physical block for every
 * member and every j < ceil(P_i / block_size).
 *   workspace     >= paged_attn_decode_shared_workspace_size(...) bytes; same
 *                 contract as paged_attn_decode_multi
 * Two launches on `stream`; other arguments and errors as for
 * paged_attn_decode_multi.
 */
size_t paged_attn_decode_shared_workspace_size(int32_t num_seqs, int32_t num_groups,
                                               int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim);
int paged_attn_decode_shared(void *out, const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, const int32_t *context_lens,
                             const int32_t *group_starts, const int32_t *prefix_lens,
                             int32_t num_seqs, int32_t num_groups, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_context_len, float scale, int32_t dtype,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_check_inputs -- check the device-resident data the other calls take on
 * trust (a debugging aid; it reads only the arguments named here).
 *
 * Violations looked for (kinds):
 *   1  context_lens[i] outside [0, max_context_len]
 *   2  a Block Table entry a sequence uses (j < ceil(L_i / block_size)) outside
 *      [0, num_blocks); padding entries past that are never read and not checked
 *   3  a non-negative slot_mapping entry at or past num_blocks * block_size
 *   4  a non-negative slot given twice (only with a bitmap)
 *   slot_mapping  int64 [num_tokens] on the device, or NULL with num_tokens 0
 *   bitmap        device scratch of ceil(num_blocks*block_size / 32) uint32
 *                 (cleared by the call), or NULL to skip the repeat check
 *   result        int64 [4] on the device, written in stream order: the
 *                 number of violations, then the kind, index (sequence or
 *                 token) and value of one of them (kind 0 and index -1 if none)
 * Errors: PKV_ERR_SHAPE / PKV_ERR_NULL / PKV_ERR_ALIGN (pointers not aligned to
 * their element) / PKV_ERR_WORKSPACE (bitmap too small) on the host, as for the
 * other calls.  Nothing is synchronised.
 */
int paged_check_inputs(const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int64_t num_blocks, int32_t block_size,
                       int32_t max_context_len, const int64_t *slot_mapping, int64_t num_tokens,
                       uint32_t *bitmap, size_t bitmap_bytes, int64_t *result, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
