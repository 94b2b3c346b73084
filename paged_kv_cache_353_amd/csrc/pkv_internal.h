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
    int64_t num_slots;       // num_blocks * block_size: slots at or past it are skipped
    int64_t k_token_stride;  // elements
    int64_t v_token_stride;  // elements
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t elem_bytes;
};

hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- block copy
struct CopyBlocksArgs {
    void *k_cache;
    void *v_cache;
    const int64_t *pairs;  // [num_pairs][2] (src, dst); a negative entry skips the pair
    int64_t num_pairs;
    int64_t block_bytes;   // num_kv_heads * block_size * head_dim * elem_bytes
};

hipError_t launch_copy_blocks(const CopyBlocksArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- append at L - 1
// The token of each sequence written to position context_len - 1 (the slot
// looked up in the Block Table); used ahead of a decode that cannot append.
struct AppendLastArgs {
    const void *k_new;            // [num_seqs][num_kv_heads][head_dim]
    const void *v_new;
    void *k_cache;
    void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int32_t elem_bytes;
};

hipError_t launch_append_last(const AppendLastArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- input checks
struct CheckArgs {
    const int32_t *block_tables;
    const int32_t *context_lens;
    const int64_t *slot_mapping;   // may be null
    uint32_t *bitmap;              // one bit per slot, may be null (no repeat check)
    int64_t *result;               // [4]: violations, kind, index, value
    int64_t bitmap_words;
    int64_t num_tokens;
    int64_t num_blocks;
    int32_t num_seqs;
    int32_t max_blocks_per_seq;
    int32_t block_size;
    int32_t max_context_len;
};

hipError_t launch_check(const CheckArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- decode
constexpr int kWavesPerGroup = 4;   // independent waves per workgroup
constexpr int kWavesPerSimd = 1;    // resident waves per SIMD the grid is sized for (at most)
// Dynamic LDS reserved (and not used) by each one-query decode workgroup, so
// that a CU (160 KiB of LDS) holds one of them: four waves, one per SIMD.
// The kernel's registers would let two share a SIMD, and then the older wave
// of each SIMD takes the memory pipeline while the younger one's equal share
// finishes long after it.
constexpr unsigned kDecodeLdsPin = 96u * 1024u;
constexpr int kMaxWaves = 8192;     // 256 CUs x 32 resident waves; sizes the workspace
// Arrival counters sit in a region of fixed size at the start of every
// workspace, so that partial results written by a call of one shape never
// land where a later call of another shape expects zeroed counters.
constexpr int64_t kMaxUnits = (int64_t)1 << 20;   // num_seqs * num_kv_heads

struct DecodeArgs {
    void *out;
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    // fused step only (null otherwise): the appended tokens [num_seqs][num_kv_heads][head_dim]
    // and the caches again, writable, for their slots
    const void *k_new;
    const void *v_new;
    void *k_cache_w;
    void *v_cache_w;
    int32_t *ws_cnt;   // [kMaxUnits] per-unit arrival counters, zero between calls
    int32_t *ws_gcnt;  // [kMaxWaves + kMaxUnits] per-group arrival counters, zero between calls
    float *ws_acc;     // [kMaxWaves + units][group][head_dim] partial outputs (one per segment)
    float *ws_ml;      // [kMaxWaves + units][group][2]        (max, exp-sum) of each
    float *ws_gacc;    // [kMaxWaves + units][group][head_dim] merged groups of segments
    float *ws_gml;     // [kMaxWaves + units][group][2]
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int32_t num_waves;  // waves in the grid (multiple of kWavesPerGroup, <= kMaxWaves)
    float scale_log2;   // scale * log2(e): scores are kept in base-2 exponent units
};

// Workspace layout for these sizes; offsets and total in bytes.  The
// counters come first, in a region whose size does not depend on the sizes.
constexpr size_t kCounterBytes = ((size_t)kMaxUnits + (size_t)kMaxWaves + (size_t)kMaxUnits) * sizeof(int32_t);
static_assert(kCounterBytes % 256 == 0, "partial results start 256-byte aligned");
struct DecodeWorkspace {
    size_t cnt_offset;
    size_t gcnt_offset;
    size_t acc_offset;
    size_t ml_offset;
    size_t gacc_offset;
    size_t gml_offset;
    size_t bytes;
};

inline DecodeWorkspace decode_workspace(int32_t num_seqs, int32_t num_kv_heads, int32_t group,
                                        int32_t head_dim) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t units = (size_t)num_seqs * (size_t)num_kv_heads;
    const size_t slots = (size_t)kMaxWaves + units;
    const size_t acc_bytes = up(slots * (size_t)group * (size_t)head_dim * sizeof(float));
    const size_t ml_bytes = up(slots * (size_t)group * 2 * sizeof(float));
    DecodeWorkspace w{};
    w.cnt_offset = 0;
    w.gcnt_offset = (size_t)kMaxUnits * sizeof(int32_t);
    w.acc_offset = up(kCounterBytes);
    w.ml_offset = w.acc_offset + acc_bytes;
    w.gacc_offset = w.ml_offset + ml_bytes;
    w.gml_offset = w.gacc_offset + acc_bytes;
    w.bytes = w.gml_offset + ml_bytes;
    return w;
}

// A fixed scratch area per GPU (a static device array) for the decode step
// that allocates nothing.  Its counter region has a fixed place and size so
// that the records of one call never land on the counters of another.
constexpr int64_t kStaticMaxUnits = 16384;   // num_seqs * num_kv_heads
constexpr int64_t kStaticMaxWaves = 1024;    // waves of the decode grid
constexpr size_t kStaticScratchBytes = (size_t)24 << 20;
constexpr size_t kStaticCounterBytes =
    (((size_t)(kStaticMaxUnits + kStaticMaxWaves + kStaticMaxUnits) * sizeof(int32_t)) + 255) & ~(size_t)255;
struct StaticScratchLayout {
    size_t cnt_offset, gcnt_offset, acc_offset, ml_offset, gacc_offset, gml_offset, bytes;
    bool fits;
};
inline StaticScratchLayout static_scratch_layout(int32_t num_seqs, int32_t num_kv_heads, int32_t group,
                                                 int32_t head_dim, int64_t waves) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int64_t units = (int64_t)num_seqs * num_kv_heads;
    const size_t slots = (size_t)waves + (size_t)units;
    const size_t acc_bytes = up(slots * (size_t)group * (size_t)head_dim * sizeof(float));
    const size_t ml_bytes = up(slots * (size_t)group * 2 * sizeof(float));
    StaticScratchLayout l{};
    l.cnt_offset = 0;
    l.gcnt_offset = (size_t)kStaticMaxUnits * sizeof(int32_t);
    l.acc_offset = kStaticCounterBytes;
    l.ml_offset = l.acc_offset + acc_bytes;
    l.gacc_offset = l.ml_offset + ml_bytes;
    l.gml_offset = l.gacc_offset + acc_bytes;
    l.bytes = l.gml_offset + ml_bytes;
    l.fits = units <= kStaticMaxUnits && waves <= kStaticMaxWaves && l.bytes <= kStaticScratchBytes;
    return l;
}
// Device address of this GPU's scratch array (looked up once per device, its
// counter region cleared on the given stream at that first use), or null.
void *static_scratch(int device, hipStream_t stream);

bool decode_supported(int32_t dtype, int32_t head_dim, int32_t group);

// Bytes of per-lane scratch (register spills) of the one-query kernel for this
// configuration; a configuration that spills is routed to the many-column
// kernel instead (0 on error).
int decode_scratch_bytes(int32_t dtype, int32_t head_dim, int32_t group);

// Resident waves per CU of the decode kernel for this configuration (0 on error).
int decode_waves_per_cu(int32_t dtype, int32_t head_dim, int32_t group);

// dtype: 0 f32, 1 f16, 2 bf16.
hipError_t launch_attn_decode(int32_t dtype, int32_t head_dim, int32_t group,
                              const DecodeArgs &a, hipStream_t stream);

// ------------------------------------------------ many query columns per KV head
// One kernel serves two call kinds.  A row is a sequence or a group of
// sequences; each of its (KV head, column chunks) units streams the row's
// tokens once for up to kMultiCols * kMultiChunksMax query columns.
enum MultiMode : int32_t {
    kModeMulti = 0,   // rows = sequences; columns = (query token, head), causal among the new tokens
    kModeShared = 1,  // rows = the groups' shared prefixes [0, P), columns = (member, head), then the
                      // sequences' suffixes [P, L), columns = heads; a reduce pass merges the two
};
constexpr int kMultiCols = 16;      // query columns per chunk (the MFMA's N)
constexpr int kMultiChunksMax = 2;  // column chunks a unit streams together (one K/V load)
// Resident waves per SIMD the many-column grid is sized for.  With two, the
// younger wave of each SIMD streams at about 60% of the older one's rate and
// the call ends on its tail; one wave per SIMD measured 15-25% faster.
constexpr int kMultiWavesPerSimd = 1;

struct MultiArgs {
    void *out;
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    const int32_t *group_starts;  // shared mode: [num_groups + 1]
    const int32_t *prefix_lens;   // shared mode: [num_seqs]
    int32_t *unit_desc;           // multi mode: [0] units of the call; then 8 int32 per unit (from
                                  // word 8): first record slot, records, row, (KV head << 16) | chunk,
                                  // table sequence, columns, first attended position, 0
    int32_t *col_desc;            // shared mode: 4 int32 per (sequence, q head), suffix part then
                                  // prefix part: first record slot, records, column, flags
    float *ws_acc;                // [kMaxWaves + units][columns of a unit][head_dim] partial records
    float *ws_ml;                 // [kMaxWaves + units][columns of a unit][2]
    int32_t mode;
    int32_t num_rows;             // multi: sequences; shared: groups + sequences
    int32_t num_seqs;
    int32_t num_groups;           // shared mode
    int32_t max_units;            // units the workspace holds
    int32_t num_query_tokens;     // multi mode (1 otherwise)
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t block_shift;          // log2(block_size)
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int32_t num_waves;
    float scale_log2;
};

// Workspace of the many-column kernels.  The counter region of the
// single-query decode is left in place (and untouched), so one workspace can
// serve both kinds of call.
struct MultiWorkspace {
    size_t desc_offset;      // unit descriptors (multi)
    size_t col_desc_offset;  // column descriptors (shared)
    size_t acc_offset;       // partial records
    size_t ml_offset;
    size_t bytes;
};

inline MultiWorkspace multi_workspace(int64_t max_units, int64_t items, int32_t head_dim) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t slots = (size_t)kMaxWaves + (size_t)max_units;
    const size_t cols = (size_t)kMultiCols * kMultiChunksMax;   // a record holds every column of a unit
    MultiWorkspace w{};
    w.desc_offset = up(kCounterBytes);
    w.col_desc_offset = w.desc_offset + up((8 + 8 * (size_t)max_units) * sizeof(int32_t));
    w.acc_offset = w.col_desc_offset + up(2 * 4 * (size_t)items * sizeof(int32_t));
    w.ml_offset = w.acc_offset + up(slots * cols * (size_t)head_dim * sizeof(float));
    w.bytes = w.ml_offset + up(slots * cols * 2 * sizeof(float));
    return w;
}

bool multi_supported(int32_t dtype, int32_t head_dim);
int multi_waves_per_cu(int32_t dtype, int32_t head_dim, int32_t chunks);
// chunks: column chunks per unit (1 or 2), chosen by the caller from the columns a row has
hipError_t launch_attn_multi(int32_t dtype, int32_t head_dim, int32_t chunks, const MultiArgs &a,
                             hipStream_t stream);

}  // namespace pkv
