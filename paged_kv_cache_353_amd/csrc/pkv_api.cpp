// C ABI of libpkv.so: host-side argument checks, work planning and launches.
// Every check here runs on the host before anything is queued; nothing reads
// device memory or synchronises.
#include "pkv.h"

#include <atomic>
#include <cmath>

#include "pkv_internal.h"

static_assert(pkv::kCounterBytes == PKV_DECODE_COUNTER_BYTES, "header and library agree on the counter region");

namespace {

constexpr int kVersion = 200;  // 0.2.0: one-launch decode, counter region in the workspace

int elem_bytes(int32_t dtype) {
    switch (dtype) {
        case PKV_F32: return 4;
        case PKV_F16: return 2;
        case PKV_BF16: return 2;
        default: return 0;
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device, asked once per device: the attribute
// query costs more than the launch it sizes.
constexpr int kMaxDevices = 64;
int current_device_cus(int *device_out) {
    static std::atomic<int> cache[kMaxDevices];
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return 0;
    if (device_out) *device_out = device;
    if (device < 0 || device >= kMaxDevices) {
        int cus = 0;
        return hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess ? cus : 0;
    }
    int cus = cache[device].load(std::memory_order_relaxed);
    if (cus > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
    cache[device].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace

extern "C" {

const char *pkv_status_string(int status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_NULL: return "a required pointer is NULL";
        case PKV_ERR_SHAPE: return "a size is out of range or sizes disagree";
        case PKV_ERR_DTYPE: return "unknown dtype code";
        case PKV_ERR_UNSUPPORTED: return "no kernel is built for this head_dim / block_size / head group";
        case PKV_ERR_WORKSPACE: return "workspace missing or smaller than paged_attn_decode_workspace_size()";
        case PKV_ERR_ALIGN: return "a pointer or token stride is not 16-byte aligned";
        case PKV_ERR_HIP: return "the HIP runtime reported an error at launch";
        default: return "unknown status";
    }
}

int pkv_version(void) { return kVersion; }

int paged_kv_write(const void *k, const void *v, void *k_cache, void *v_cache,
                   const int64_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   int64_t k_token_stride, int64_t v_token_stride, int32_t dtype,
                   hipStream_t stream) {
    const int eb = elem_bytes(dtype);
    if (eb == 0) return PKV_ERR_DTYPE;
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return PKV_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (k_token_stride < row || v_token_stride < row) return PKV_ERR_SHAPE;
    if (num_tokens == 0) return PKV_OK;
    if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (k_token_stride * eb) % 16 != 0 || (v_token_stride * eb) % 16 != 0)
        return PKV_ERR_ALIGN;
    if (num_tokens > ((int64_t)1 << 40) / row) return PKV_ERR_SHAPE;
    pkv::KvWriteArgs a{};
    a.k = k;
    a.v = v;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_slots = num_blocks * (int64_t)block_size;
    a.k_token_stride = k_token_stride;
    a.v_token_stride = v_token_stride;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.elem_bytes = eb;
    return pkv::launch_kv_write(a, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_pairs,
                      int64_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int64_t num_blocks, int32_t dtype,
                      hipStream_t stream) {
    const int eb = elem_bytes(dtype);
    if (eb == 0) return PKV_ERR_DTYPE;
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return PKV_ERR_SHAPE;
    if (num_pairs > 0x7FFFFFFF) return PKV_ERR_SHAPE;
    if (num_pairs == 0) return PKV_OK;
    if (!k_cache || !v_cache || !block_pairs) return PKV_ERR_NULL;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * eb;
    if (!aligned16(k_cache) || !aligned16(v_cache) || block_bytes % 16 != 0) return PKV_ERR_ALIGN;
    pkv::CopyBlocksArgs a{};
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.pairs = block_pairs;
    a.num_pairs = num_pairs;
    a.block_bytes = block_bytes;
    return pkv::launch_copy_blocks(a, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_check_inputs(const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int64_t num_blocks, int32_t block_size,
                       int32_t max_context_len, const int64_t *slot_mapping, int64_t num_tokens,
                       uint32_t *bitmap, size_t bitmap_bytes, int64_t *result, hipStream_t stream) {
    if (num_seqs < 0 || num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || max_context_len < 0 ||
        (num_seqs > 0 && max_blocks_per_seq <= 0))
        return PKV_ERR_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size < max_context_len) return PKV_ERR_SHAPE;
    if (!result) return PKV_ERR_NULL;
    if (num_seqs > 0 && (!block_tables || !context_lens)) return PKV_ERR_NULL;
    if (num_tokens > 0 && !slot_mapping) return PKV_ERR_NULL;
    auto misaligned = [](const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; };
    if (misaligned(result, 8) || misaligned(slot_mapping, 8) || misaligned(bitmap, 4) ||
        misaligned(block_tables, 4) || misaligned(context_lens, 4))
        return PKV_ERR_ALIGN;
    const int64_t slots = num_blocks * (int64_t)block_size;
    if (bitmap && bitmap_bytes < (size_t)((slots + 31) / 32) * 4) return PKV_ERR_WORKSPACE;
    pkv::CheckArgs a{};
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.slot_mapping = num_tokens > 0 ? slot_mapping : nullptr;
    a.bitmap = bitmap;
    a.bitmap_words = bitmap ? (slots + 31) / 32 : 0;
    a.result = result;
    a.num_tokens = num_tokens;
    a.num_blocks = num_blocks;
    a.num_seqs = num_seqs;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.block_size = block_size;
    a.max_context_len = max_context_len;
    return pkv::launch_check(a, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_context_len) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_context_len < 0 || num_q_heads % num_kv_heads != 0 ||
        (int64_t)num_seqs * num_kv_heads > pkv::kMaxUnits)
        return 0;
    const int32_t group = num_q_heads / num_kv_heads;
    const size_t one = pkv::decode_workspace(num_seqs, num_kv_heads, group, head_dim).bytes;
    // enough for the many-column kernel too, which serves the group sizes the
    // one-query kernel does not (or would only serve with register spills)
    const int64_t units = (int64_t)num_seqs * num_kv_heads * ((group + pkv::kMultiCols - 1) / pkv::kMultiCols);
    if (units > pkv::kMaxUnits) return one;
    const size_t many = pkv::multi_workspace(units, 0, head_dim).bytes;
    return one > many ? one : many;
}

}  // extern "C"

namespace {

// One query per sequence through the many-column kernel (T = 1), after the
// appended tokens are written (fused step); defined with the other
// many-column entry points below.
int decode_through_multi(void *out, const void *q, const void *k_new, const void *v_new,
                         const void *k_cache, const void *v_cache, const int32_t *block_tables,
                         const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                         float scale, int32_t dtype, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

// Where a decode call keeps its arrival counters and partial records.
struct DecodeScratch {
    int32_t *cnt;
    int32_t *gcnt;
    float *acc;
    float *ml;
    float *gacc;
    float *gml;
};

// Host checks of a one-query decode call; sets *one_query to whether the
// one-query kernel serves it (the others go to the many-column kernel).
int decode_checks(const void *out, const void *q, const void *k_new, const void *v_new, const void *k_cache,
                  const void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                  int32_t max_context_len, float scale, int32_t dtype, bool *one_query) {
    if (elem_bytes(dtype) == 0) return PKV_ERR_DTYPE;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0)
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size < max_context_len) return PKV_ERR_SHAPE;
    if (num_seqs > 65535 || num_kv_heads > 65535) return PKV_ERR_SHAPE;
    if ((int64_t)num_seqs * num_kv_heads > pkv::kMaxUnits) return PKV_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
    const int32_t group = num_q_heads / num_kv_heads;
    // The one-query kernel serves group sizes 1, 2, 4 and 8 where it keeps
    // its state in registers; other group sizes, and configurations whose
    // compiled kernel would spill (none at present; a spilling build ran
    // about ten times slower), go to the many-column kernel.
    *one_query = pkv::decode_supported(dtype, head_dim, group) && block_size % 16 == 0 && block_size <= 256 &&
                 !(num_seqs > 0 && pkv::decode_scratch_bytes(dtype, head_dim, group) > 0);
    if (!*one_query) return PKV_OK;
    // sub-tile indices of the whole batch are kept in 32 bits
    if ((int64_t)num_seqs * num_kv_heads * (((int64_t)max_context_len + 15) / 16) >= ((int64_t)1 << 31))
        return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_NULL;
    if ((k_new == nullptr) != (v_new == nullptr)) return PKV_ERR_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_ALIGN;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_ALIGN;
    return PKV_OK;
}

// Waves of the one-query decode grid: as many as the GPU holds at once (0 on error).
int64_t decode_grid_waves(int32_t dtype, int32_t head_dim, int32_t group) {
    const int cus = current_device_cus(nullptr);
    int per_cu = pkv::decode_waves_per_cu(dtype, head_dim, group);
    if (per_cu <= 0 || cus <= 0) return 0;
    per_cu = per_cu < 4 * pkv::kWavesPerSimd ? per_cu : 4 * pkv::kWavesPerSimd;
    int64_t waves = (int64_t)cus * per_cu;
    waves = waves < pkv::kMaxWaves ? waves : pkv::kMaxWaves;
    return waves - waves % pkv::kWavesPerGroup;
}

int decode_launch(void *out, const void *q, const void *k_new, const void *v_new, const void *k_cache,
                  const void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                  int32_t dtype, int64_t waves, const DecodeScratch &s, hipStream_t stream) {
    pkv::DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.k_new = k_new;
    a.v_new = v_new;
    // the fused step writes the appended token into the caches it was given
    a.k_cache_w = const_cast<void *>(k_cache);
    a.v_cache_w = const_cast<void *>(v_cache);
    a.ws_cnt = s.cnt;
    a.ws_gcnt = s.gcnt;
    a.ws_acc = s.acc;
    a.ws_ml = s.ml;
    a.ws_gacc = s.gacc;
    a.ws_gml = s.gml;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.num_waves = (int32_t)waves;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    return pkv::launch_attn_decode(dtype, head_dim, num_q_heads / num_kv_heads, a, stream) == hipSuccess
               ? PKV_OK
               : PKV_ERR_HIP;
}

// Shared by paged_attn_decode (k_new == v_new == NULL) and paged_decode_step.
int decode_impl(void *out, const void *q, const void *k_new, const void *v_new,
                const void *k_cache, const void *v_cache, const int32_t *block_tables,
                const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                float scale, int32_t dtype, void *workspace, size_t workspace_bytes,
                hipStream_t stream) {
    bool one_query = false;
    int st = decode_checks(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, num_seqs,
                           num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                           max_context_len, scale, dtype, &one_query);
    if (st != PKV_OK) return st;
    if (!one_query)
        return decode_through_multi(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                    max_blocks_per_seq, num_blocks, max_context_len, scale, dtype, workspace,
                                    workspace_bytes, stream);
    if (num_seqs == 0) return PKV_OK;
    const int32_t group = num_q_heads / num_kv_heads;
    const pkv::DecodeWorkspace ws = pkv::decode_workspace(num_seqs, num_kv_heads, group, head_dim);
    if (!workspace || workspace_bytes < ws.bytes) return PKV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PKV_ERR_ALIGN;
    const int64_t waves = decode_grid_waves(dtype, head_dim, group);
    if (waves <= 0) return PKV_ERR_HIP;
    char *w = static_cast<char *>(workspace);
    const DecodeScratch s{reinterpret_cast<int32_t *>(w + ws.cnt_offset), reinterpret_cast<int32_t *>(w + ws.gcnt_offset),
                          reinterpret_cast<float *>(w + ws.acc_offset), reinterpret_cast<float *>(w + ws.ml_offset),
                          reinterpret_cast<float *>(w + ws.gacc_offset), reinterpret_cast<float *>(w + ws.gml_offset)};
    return decode_launch(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, num_seqs,
                         num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len,
                         scale, dtype, waves, s, stream);
}

// Units of the multi-query kernel for these sizes (an upper bound in the
// shared-prefix case, where group sizes live on the device).
int64_t multi_units(int32_t num_seqs, int32_t num_query_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads) {
    const int64_t cols = (int64_t)num_query_tokens * (num_q_heads / num_kv_heads);
    return (int64_t)num_seqs * num_kv_heads * ((cols + pkv::kMultiCols - 1) / pkv::kMultiCols);
}
int64_t shared_units(int32_t num_seqs, int32_t num_groups, int32_t num_q_heads, int32_t num_kv_heads) {
    const int64_t G = num_q_heads / num_kv_heads;
    // prefix rows: sum over groups of ceil(members * G / 16) <= ceil(S * G / 16) + groups;
    // suffix rows: ceil(G / 16) per (sequence, KV head); one launch holds both
    const int64_t pre = (int64_t)num_kv_heads * (((int64_t)num_seqs * G + pkv::kMultiCols - 1) / pkv::kMultiCols +
                                                 num_groups);
    const int64_t suf = (int64_t)num_seqs * num_kv_heads * ((G + pkv::kMultiCols - 1) / pkv::kMultiCols);
    return pre + suf;
}

int log2_exact(int32_t x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return (1 << s) == x ? s : -1;
}

// Host checks shared by the multi-query entry points.
int multi_checks(const void *out, const void *q, const void *k_cache, const void *v_cache,
                 const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                 int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len, float scale,
                 int32_t dtype, int64_t units) {
    if (elem_bytes(dtype) == 0) return PKV_ERR_DTYPE;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0)
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size < max_context_len) return PKV_ERR_SHAPE;
    if (num_seqs > 65535 || num_kv_heads > 65535 || num_q_heads > 65535) return PKV_ERR_SHAPE;
    if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
    if (!pkv::multi_supported(dtype, head_dim)) return PKV_ERR_UNSUPPORTED;
    const int bsh = log2_exact(block_size);
    if (bsh < 4 || bsh > 8) return PKV_ERR_UNSUPPORTED;   // 16 .. 256 tokens, a power of two
    if (units > pkv::kMaxUnits) return PKV_ERR_UNSUPPORTED;
    // sub-tile indices of the whole call are kept in 32 bits
    if (units * (((int64_t)max_context_len + 15) / 16 + 1) >= ((int64_t)1 << 31)) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_ALIGN;
    return PKV_OK;
}

// Column chunks a unit streams together: two when rows have more than 16
// query columns per KV head (each K/V tile is then loaded once for 32).
int32_t chunks_for(int64_t cols) { return cols > pkv::kMultiCols ? 2 : 1; }

int multi_waves(int32_t dtype, int32_t head_dim, int32_t chunks, int64_t *waves) {
    const int cus = current_device_cus(nullptr);
    int per_cu = pkv::multi_waves_per_cu(dtype, head_dim, chunks);
    if (per_cu <= 0 || cus <= 0) return PKV_ERR_HIP;
    per_cu = per_cu < 4 * pkv::kMultiWavesPerSimd ? per_cu : 4 * pkv::kMultiWavesPerSimd;
    int64_t w = (int64_t)cus * per_cu;
    w = w < pkv::kMaxWaves ? w : pkv::kMaxWaves;
    w -= w % pkv::kWavesPerGroup;
    *waves = w;
    return PKV_OK;
}

void fill_multi_split(pkv::MultiArgs &a, const pkv::MultiWorkspace &ws, void *workspace) {
    char *w = static_cast<char *>(workspace);
    a.unit_desc = reinterpret_cast<int32_t *>(w + ws.desc_offset);
    a.col_desc = reinterpret_cast<int32_t *>(w + ws.col_desc_offset);
    a.ws_acc = reinterpret_cast<float *>(w + ws.acc_offset);
    a.ws_ml = reinterpret_cast<float *>(w + ws.ml_offset);
}

int decode_through_multi(void *out, const void *q, const void *k_new, const void *v_new,
                         const void *k_cache, const void *v_cache, const int32_t *block_tables,
                         const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                         float scale, int32_t dtype, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    const int64_t units = multi_units(num_seqs, 1, num_q_heads, num_kv_heads);
    int st = multi_checks(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                          num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len,
                          scale, dtype, units);
    if (st != PKV_OK || num_seqs == 0) return st;
    if ((k_new == nullptr) != (v_new == nullptr)) return PKV_ERR_NULL;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_ALIGN;
    const pkv::MultiWorkspace ws = pkv::multi_workspace(units, 0, head_dim);
    if (!workspace || workspace_bytes < ws.bytes) return PKV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PKV_ERR_ALIGN;
    const int32_t chunks = chunks_for(num_q_heads / num_kv_heads);
    int64_t waves = 0;
    if ((st = multi_waves(dtype, head_dim, chunks, &waves)) != PKV_OK) return st;
    if (k_new) {
        // the appended token of each sequence first, at position L - 1
        pkv::AppendLastArgs ap{};
        ap.k_new = k_new;
        ap.v_new = v_new;
        ap.k_cache = const_cast<void *>(k_cache);
        ap.v_cache = const_cast<void *>(v_cache);
        ap.block_tables = block_tables;
        ap.context_lens = context_lens;
        ap.num_seqs = num_seqs;
        ap.num_kv_heads = num_kv_heads;
        ap.head_dim = head_dim;
        ap.block_size = block_size;
        ap.max_blocks_per_seq = max_blocks_per_seq;
        ap.max_context_len = max_context_len;
        ap.elem_bytes = elem_bytes(dtype);
        if (pkv::launch_append_last(ap, stream) != hipSuccess) return PKV_ERR_HIP;
    }
    pkv::MultiArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    fill_multi_split(a, ws, workspace);
    a.mode = pkv::kModeMulti;
    a.num_rows = num_seqs;
    a.num_seqs = num_seqs;
    a.max_units = (int32_t)units;
    a.num_query_tokens = 1;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_shift = log2_exact(block_size);
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.num_waves = (int32_t)waves;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    return pkv::launch_attn_multi(dtype, head_dim, chunks, a, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

extern "C" {

size_t paged_attn_decode_multi_workspace_size(int32_t num_seqs, int32_t num_query_tokens,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim) {
    if (num_seqs <= 0 || num_query_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        num_q_heads % num_kv_heads != 0 || num_seqs > 65535 || num_query_tokens > 65535)
        return 0;
    const int64_t units = multi_units(num_seqs, num_query_tokens, num_q_heads, num_kv_heads);
    if (units > pkv::kMaxUnits) return 0;
    return pkv::multi_workspace(units, 0, head_dim).bytes;
}

int paged_attn_decode_multi(void *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                            int32_t num_query_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                            int64_t num_blocks, int32_t max_context_len, float scale, int32_t dtype,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (num_query_tokens <= 0 || num_query_tokens > 65535) return PKV_ERR_SHAPE;
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (num_seqs < 0) return PKV_ERR_SHAPE;
    const int64_t units = multi_units(num_seqs, num_query_tokens, num_q_heads, num_kv_heads);
    int st = multi_checks(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                          num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len,
                          scale, dtype, units);
    if (st != PKV_OK || num_seqs == 0) return st;
    const pkv::MultiWorkspace ws = pkv::multi_workspace(units, 0, head_dim);
    if (!workspace || workspace_bytes < ws.bytes) return PKV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PKV_ERR_ALIGN;
    const int32_t chunks = chunks_for((int64_t)num_query_tokens * (num_q_heads / num_kv_heads));
    int64_t waves = 0;
    if ((st = multi_waves(dtype, head_dim, chunks, &waves)) != PKV_OK) return st;
    pkv::MultiArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    fill_multi_split(a, ws, workspace);
    a.mode = pkv::kModeMulti;
    a.num_rows = num_seqs;
    a.num_seqs = num_seqs;
    a.max_units = (int32_t)units;
    a.num_query_tokens = num_query_tokens;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_shift = log2_exact(block_size);
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.num_waves = (int32_t)waves;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    return pkv::launch_attn_multi(dtype, head_dim, chunks, a, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

size_t paged_attn_decode_shared_workspace_size(int32_t num_seqs, int32_t num_groups, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim) {
    if (num_seqs <= 0 || num_groups <= 0 || num_groups > num_seqs || num_q_heads <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || num_q_heads % num_kv_heads != 0 || num_seqs > 65535)
        return 0;
    const int64_t units = shared_units(num_seqs, num_groups, num_q_heads, num_kv_heads);
    if (units > pkv::kMaxUnits) return 0;
    return pkv::multi_workspace(units, (int64_t)num_seqs * num_q_heads, head_dim).bytes;
}

int paged_attn_decode_shared(void *out, const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, const int32_t *context_lens,
                             const int32_t *group_starts, const int32_t *prefix_lens, int32_t num_seqs,
                             int32_t num_groups, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_context_len, float scale, int32_t dtype, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (num_seqs < 0 || num_groups < 0 || num_groups > num_seqs || (num_seqs > 0 && num_groups == 0))
        return PKV_ERR_SHAPE;
    const int64_t units = shared_units(num_seqs, num_groups, num_q_heads, num_kv_heads);
    int st = multi_checks(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                          num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len,
                          scale, dtype, units);
    if (st != PKV_OK || num_seqs == 0) return st;
    if (!group_starts || !prefix_lens) return PKV_ERR_NULL;
    const pkv::MultiWorkspace ws = pkv::multi_workspace(units, (int64_t)num_seqs * num_q_heads, head_dim);
    if (!workspace || workspace_bytes < ws.bytes) return PKV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PKV_ERR_ALIGN;
    // prefix rows have (members x group) columns: the mean group size decides
    const int64_t G = num_q_heads / num_kv_heads;
    const int32_t chunks = chunks_for(((int64_t)num_seqs * G + num_groups - 1) / num_groups);
    int64_t waves = 0;
    if ((st = multi_waves(dtype, head_dim, chunks, &waves)) != PKV_OK) return st;
    pkv::MultiArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.group_starts = group_starts;
    a.prefix_lens = prefix_lens;
    fill_multi_split(a, ws, workspace);
    a.num_query_tokens = 1;
    a.num_seqs = num_seqs;
    a.max_units = (int32_t)units;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_shift = log2_exact(block_size);
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    // one pass streams every group's shared prefix once for all its members
    // and every sequence's own suffix; the reduce pass merges the two parts
    a.mode = pkv::kModeShared;
    a.num_groups = num_groups;
    a.num_rows = num_groups + num_seqs;
    a.num_waves = (int32_t)waves;
    return pkv::launch_attn_multi(dtype, head_dim, chunks, a, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_attn_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                      int64_t num_blocks, int32_t max_context_len, float scale,
                      int32_t dtype, void *workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks, max_context_len, scale, dtype, workspace,
                       workspace_bytes, stream);
}

int paged_decode_step_static(void *out, const void *q, const void *k_new, const void *v_new,
                             void *k_cache, void *v_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                             float scale, int32_t dtype, hipStream_t stream) {
    if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_NULL;
    bool one_query = false;
    int st = decode_checks(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, num_seqs,
                           num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                           max_context_len, scale, dtype, &one_query);
    if (st != PKV_OK) return st;
    if (!one_query) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    const int32_t group = num_q_heads / num_kv_heads;
    const int64_t waves = decode_grid_waves(dtype, head_dim, group);
    if (waves <= 0) return PKV_ERR_HIP;
    // the layout must fit the fixed array: counters in their fixed region,
    // records of this call's sizes after it
    const pkv::StaticScratchLayout lay = pkv::static_scratch_layout(num_seqs, num_kv_heads, group, head_dim, waves);
    if (!lay.fits) return PKV_ERR_WORKSPACE;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return PKV_ERR_HIP;
    char *w = static_cast<char *>(pkv::static_scratch(device, stream));
    if (!w) return PKV_ERR_HIP;
    const DecodeScratch s{reinterpret_cast<int32_t *>(w + lay.cnt_offset),
                          reinterpret_cast<int32_t *>(w + lay.gcnt_offset),
                          reinterpret_cast<float *>(w + lay.acc_offset), reinterpret_cast<float *>(w + lay.ml_offset),
                          reinterpret_cast<float *>(w + lay.gacc_offset),
                          reinterpret_cast<float *>(w + lay.gml_offset)};
    return decode_launch(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, num_seqs,
                         num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len,
                         scale, dtype, waves, s, stream);
}

int paged_decode_step(void *out, const void *q, const void *k_new, const void *v_new,
                      void *k_cache, void *v_cache, const int32_t *block_tables,
                      const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                      float scale, int32_t dtype, void *workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_NULL;
    return decode_impl(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks, max_context_len, scale, dtype, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"
