// Paged decode attention with many query columns per KV head, for gfx950.
//
// Two extensions of the single-query decode share this kernel:
//  * several query tokens per sequence (parallel sampling, beam search and
//    draft verification produce them), each attending to every position up
//    to its own: the new tokens are the last T positions of the sequence;
//  * forks whose Block Tables point at the same physical blocks for a common
//    prefix ("PagedAttention核心思想" section 2.4.3): the prefix of a group is
//    streamed once for the query heads of all its members, each member's own
//    suffix separately, and the two partial results are merged.
// Either way one K/V tile serves up to 16 query columns per chunk (two
// chunks per unit), which turns both products of the tile into matrix-core
// work:
//  * scores S = K q^T: one 16x16x32 MFMA per 32 dims, tokens as rows and
//    query columns as columns (lane (r, j) receives tokens 4r..4r+3 of
//    column j);
//  * output O^T += V^T P: one 16x16x16 MFMA per 16 output dims (two for
//    bfloat16, whose probabilities go in as head + remainder).  The B
//    operand (16 tokens x 16 columns) is exactly the score layout, rounded to
//    the cache's 16-bit type; the A operand (16 dims x 16 tokens) is taken
//    from V rows 4r..4r+3 that lane (r, c) loaded, dims c*DL..c*DL+DL-1, by
//    pairing the same element of the four rows.  Lane (r, j) ends up owning
//    dims [r*D/4, (r+1)*D/4) of column j.
// Softmax keeps one running (reference, exp-sum) per column.  The reference is
// raised lazily, only when a score exceeds it by more than 8 in base-2 units,
// so most sub-tiles need no exchange between the lanes of a column.
//
// Work split and masking follow the single-query kernel: every (row, KV head,
// column chunks) unit is cut into 16-token sub-tiles, and all sub-tiles are
// shared out in equal contiguous ranges, one per resident wave.  Units split
// between waves, and in the shared-prefix case every unit, leave partial
// records; a second, short launch merges them in a fixed order with every
// record of an output in flight at once.  K and V are streamed with the
// non-temporal policy (read once, kept out of the way of the records and
// tables in the caches).  Loads use descriptors that span
// only the unit's valid rows, so rows past the end read as zero, and every
// score outside a column's window is set to -inf before the exponential, so
// stale cache contents never reach the result.
#include "pkv_device.h"

#include <atomic>

namespace pkv {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kMDepth = 2;        // sub-tiles in flight per wave
constexpr int kDescWords = 8;     // unit descriptor: first slot, records, row, kvh|chunk, tseq, cols, lo, -
constexpr int kColDescWords = 4;  // column descriptor: first slot, records, column in the record, flags
constexpr int kHasPrefix = 1;     // flag of a suffix column descriptor: a prefix part exists
constexpr float kLazyRescale = 8.f;  // headroom of the softmax reference (weights < 2^8)
// Fixed cost of a segment (q loads, the column sums, the record), in
// sub-tiles of streaming: the split charges it to the wave whose range holds
// the start of a unit.
constexpr int kUnitCost = 4;

// Position of a wave's load or compute stage.  Every field is wave-uniform.
struct MCursor {
    int row;     // sequence, or (shared mode) group or sequence
    int kvh;     // KV head
    int chunk;   // column chunk
    int sub;     // sub-tile inside the unit
    int n;       // sub-tiles of every unit of the row
    int chunks;  // column chunks of the row
    int t0;      // position of the row's first sub-tile (a multiple of 16)
    int tend;    // one past the row's last position read
    int lo;      // first position any column of the row attends
    int L;       // the row's sequence length (multi mode: the query window's end)
    int tseq;    // sequence whose Block Table the row walks
    int cols;    // query columns of the row, per KV head
    int kind;    // kRowMulti, kRowPrefix or kRowSuffix
    int pre;     // sub-tiles of all rows before this one
    int upre;    // units of all rows before this one
};

// O^T += V^T P on one 16-dim slice: A = 4 tokens x 1 dim per lane (as four
// 16-bit values), B = the 4 probabilities of this lane's column.
template <typename DT>
__device__ __forceinline__ f32x4 mfma_pv(u32x2 a, u32x2 b, f32x4 c) {
    if constexpr (std::is_same_v<DT, BF16>) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                         __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Four probabilities as the B operand.  fp16 keeps 11 significant bits,
// enough for the output tolerance.  bfloat16 keeps 8, too few where a handful
// of tokens carry the weight, so each probability is split into a rounded
// head and the rounded remainder, and both multiply V (two MFMAs): together
// they carry about 16 significant bits.
__device__ __forceinline__ u32x2 pack_probs_f16(const float (&p)[4]) {
    f16x2 a, b;
    a[0] = (_Float16)p[0];
    a[1] = (_Float16)p[1];
    b[0] = (_Float16)p[2];
    b[1] = (_Float16)p[3];
    return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}
__device__ __forceinline__ uint32_t cvt2_bf16(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
}
__device__ __forceinline__ void split_probs_bf16(const float (&p)[4], u32x2 &hi, u32x2 &lo) {
    hi = u32x2{cvt2_bf16(p[0], p[1]), cvt2_bf16(p[2], p[3])};
    float r[4];
    static_for<0, 2>([&]<int k>() {
        r[2 * k] = p[2 * k] - as_f(hi[k] << 16);
        r[2 * k + 1] = p[2 * k + 1] - as_f(hi[k] & 0xFFFF0000u);
    });
    lo = u32x2{cvt2_bf16(r[0], r[1]), cvt2_bf16(r[2], r[3])};
}

// A lane's slice of one V row: D / 16 consecutive elements, as 32-bit words.
template <int VW>
struct VRow {
    uint32_t w[VW];
};

// 16-bit element E of a lane's slice of a V row (word E/2, half E%2).
template <int E, int VW>
__device__ __forceinline__ uint32_t v_half(const VRow<VW> &v) {
    const uint32_t w = v.w[E / 2];
    return (E & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// A row of the many-column kernel: the token range it streams, the first
// position its columns attend, its length, the sequence whose table it walks,
// its query columns per KV head and its kind.  In the shared mode rows
// [0, num_groups) are the groups' prefixes and the rest the sequences'
// suffixes.  `ld` reads a 32-bit entry of a length array (scalar or vector
// loads).
enum RowKind : int { kRowMulti = 0, kRowPrefix = 1, kRowSuffix = 2 };
struct RowInfo { int t0, tend, lo, L, tseq, cols, kind; };

template <typename LD>
__device__ __forceinline__ RowInfo row_info_of(const MultiArgs &a, int r, LD ld) {
    const int G = a.num_q_heads / a.num_kv_heads;
    const int Lmax = a.max_context_len;
    auto clampL = [&](int L) { L = L < Lmax ? L : Lmax; return L > 0 ? L : 0; };
    RowInfo ri{};
    if (a.mode == kModeShared && r < a.num_groups) {
        // members clamped to the batch (the description is device data)
        int f = ld(a.group_starts, r), e = ld(a.group_starts, r + 1);
        f = min(max(f, 0), a.num_seqs);
        e = min(max(e, f), a.num_seqs);
        const int P = f < e ? clampL(ld(a.prefix_lens, f)) : 0;
        ri.t0 = 0; ri.tend = P; ri.lo = 0; ri.L = P; ri.tseq = f; ri.cols = (e - f) * G; ri.kind = kRowPrefix;
    } else if (a.mode == kModeShared) {
        const int i = r - a.num_groups;
        const int L = clampL(ld(a.context_lens, i));
        int P = clampL(ld(a.prefix_lens, i));
        P = P < L ? P : L;
        // an empty suffix streams nothing (its output is the prefix part alone)
        ri.t0 = P < L ? (P & ~15) : P; ri.tend = L; ri.lo = P; ri.L = L; ri.tseq = i; ri.cols = G;
        ri.kind = kRowSuffix;
    } else {
        const int L = clampL(ld(a.context_lens, r));
        ri.t0 = 0; ri.tend = L; ri.lo = 0; ri.L = L; ri.tseq = r; ri.cols = a.num_query_tokens * G;
        ri.kind = kRowMulti;
    }
    return ri;
}

// Output row of column x (0-based within its row) of KV head kvh, or -1 if
// the row has no such column.  Multi mode: a row of out
// [num_seqs, num_query_tokens, Hq, D]; shared mode: the (sequence, q head)
// item, a row of out [num_seqs, Hq, D].  The query of the column is the same
// row of q.
__device__ __forceinline__ int64_t column_row(const MultiArgs &a, int row, const RowInfo &ri, int kvh, int x) {
    if (x >= ri.cols) return -1;
    const int Hq = a.num_q_heads, G = Hq / a.num_kv_heads;
    if (ri.kind == kRowMulti) {
        const int jq = x / G, h = x - jq * G;
        return ((int64_t)row * a.num_query_tokens + jq) * Hq + kvh * G + h;
    }
    if (ri.kind == kRowPrefix) {
        const int mem = x / G, h = x - mem * G;
        return (int64_t)(ri.tseq + mem) * Hq + kvh * G + h;
    }
    return (int64_t)ri.tseq * Hq + kvh * G + x;
}

template <typename DT, int D, int CH>
__global__ __launch_bounds__(kWavesPerGroup * kWave) void attn_multi_kernel(MultiArgs a) {
    constexpr int EB = DT::kBytes;
    constexpr bool kF32 = EB == 4;
    constexpr int ROW = D * EB;      // bytes per token row
    constexpr int NLK = ROW / 64;    // 16-byte K loads per lane per sub-tile
    constexpr int DL = D / 16;       // dims of a V row per lane (and output slices per sub-tile)
    constexpr int DQ = D / 4;        // output dims owned by a lane
    constexpr int VW = DL * EB / 4;  // 32-bit words of a lane's slice of a V row (2, 4 or 8)
    constexpr int UC = kMultiCols * CH;   // query columns of a unit
    constexpr int kRecFloats = UC * D;    // floats of a record's acc
    typedef VRow<VW> VReg;
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    static_assert(CH >= 1 && CH <= kMultiChunksMax, "column chunks per unit");

    const int lane = threadIdx.x & (kWave - 1);
    const int rg = lane >> 4;   // row group: tokens 4rg..4rg+3 of a sub-tile
    const int c = lane & 15;    // column within a chunk (scores, output) / token row (K) / dim slice (V)
    const int wave = uniform((int)blockIdx.x * kWavesPerGroup + (int)(threadIdx.x >> 6));
    const int R = a.num_rows, Hkv = a.num_kv_heads, Hq = a.num_q_heads;
    const int G = Hq / Hkv;
    const int Tq = a.num_query_tokens;
    const int W = a.num_waves;
    const int mode = a.mode;

    auto row_info = [&](int r, auto ld) -> RowInfo { return row_info_of(a, r, ld); };
    auto ld_vec = [](const int32_t *p, int i) { return p[i]; };
    auto ld_scalar = [](const int32_t *p, int i) { return ((const_i32_ptr)p)[i]; };
    auto tiles_of = [&](const RowInfo &ri) { return (ri.tend - ri.t0 + 15) >> 4; };
    auto chunks_of = [&](const RowInfo &ri) { return (ri.cols + UC - 1) / UC; };

    // ---- rows with nothing to stream.  Multi mode: zero outputs.  Shared
    // mode, a sequence whose suffix is empty: its column descriptors say so
    // (its result is the prefix part alone, or zero).
    for (int r = wave; r < R; r += W) {
        const RowInfo ri = row_info(r, ld_scalar);
        if (ri.tend - ri.t0 > 0 || ri.kind == kRowPrefix) continue;
        if (ri.kind == kRowMulti) {
            char *o = static_cast<char *>(a.out) + (int64_t)r * Tq * Hq * ROW;
            for (int idx = lane; idx < Tq * Hq * (ROW / 16); idx += kWave)
                *reinterpret_cast<u32x4 *>(o + (int64_t)idx * 16) = u32x4{0u, 0u, 0u, 0u};
        } else {
            typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
            for (int h = lane; h < Hq; h += kWave)
                *reinterpret_cast<i32x4 *>(a.col_desc + kColDescWords * ((int64_t)ri.tseq * Hq + h)) =
                    i32x4{0, 0, 0, ri.lo > 0 ? kHasPrefix : 0};
        }
    }

    // ---- total work and this wave's range.  In an augmented order every unit
    // is preceded by C ghost positions that stand for the fixed cost of a
    // segment; the augmented order is cut into equal ranges and a wave
    // processes the real sub-tiles of its range, so a wave whose range holds
    // unit starts streams fewer of them.  Up to kCachedBatches batches of 64
    // rows are read and scanned once, and the scans are kept for locating the
    // range; longer calls read the rows a second time.
    constexpr int kCachedBatches = 4;
    const bool cached = R <= kCachedBatches * kWave;
    int tlc[kCachedBatches], unc[kCachedBatches], inc[kCachedBatches], uinc[kCachedBatches];
    int N = 0, U = 0;
    if (cached) {
        int carry = 0, ucarry = 0;
        static_for<0, kCachedBatches>([&]<int b>() {
            tlc[b] = 0;
            unc[b] = 0;
            const int r = b * kWave + lane;
            if (r < R) {
                const RowInfo ri = row_info(r, ld_vec);
                const int n = tiles_of(ri);
                unc[b] = n > 0 ? Hkv * chunks_of(ri) : 0;
                tlc[b] = unc[b] * n;
            }
            inc[b] = carry + wave_incl_scan(tlc[b], lane);
            uinc[b] = ucarry + wave_incl_scan(unc[b], lane);
            carry = __builtin_amdgcn_readlane(inc[b], kWave - 1);
            ucarry = __builtin_amdgcn_readlane(uinc[b], kWave - 1);
        });
        N = carry;
        U = ucarry;
    } else {
        for (int base = 0; base < R; base += kWave) {
            const int r = base + lane;
            if (r < R) {
                const RowInfo ri = row_info(r, ld_vec);
                const int n = tiles_of(ri);
                N += Hkv * chunks_of(ri) * n;
                U += n > 0 ? Hkv * chunks_of(ri) : 0;
            }
        }
        N = wave_sum_i(N, lane);
        U = wave_sum_i(U, lane);
    }
    const int T = uniform(N);
    // a group description that breaks its preconditions (overlapping groups)
    // could ask for more units than the workspace holds: do nothing then
    const int units = uniform(U);
    const bool too_many = units > a.max_units;
    if (wave == 0 && lane == 0) a.unit_desc[0] = too_many ? 0 : units;   // units the reduce pass visits
    if (too_many) return;
    // Ghosts are used only when every range is longer than C, so that no
    // range holds ghosts alone and every wave gets at least one sub-tile.
    // Shared mode does without: every unit there leaves records anyway, and
    // charging its short suffix units measured slower.
    int C = mode == kModeMulti ? kUnitCost : 0;
    if (((int64_t)T + (int64_t)C * units) / W < C + 1) C = 0;
    const int64_t TA = (int64_t)T + (int64_t)C * units;   // augmented length
    const int Weff = C > 0 ? W : (T < W ? T : W);
    if (wave >= Weff) return;
    const int64_t x0 = TA * wave / Weff;                   // this wave's augmented range
    const int64_t x1 = TA * (wave + 1) / Weff;
    const bool has_end = x1 < TA;
    // the wave whose range holds augmented position x: the largest w with
    // TA * w / Weff <= x
    auto wave_of = [&](int64_t x) -> int {
        const int64_t w = ((x + 1) * Weff - 1) / TA;
        return (int)(w < Weff - 1 ? w : Weff - 1);
    };

    auto load_row = [&](MCursor &u) {
        const RowInfo ri = row_info(u.row, ld_scalar);
        u.t0 = uniform(ri.t0); u.tend = uniform(ri.tend); u.lo = uniform(ri.lo); u.L = uniform(ri.L);
        u.tseq = uniform(ri.tseq); u.cols = uniform(ri.cols); u.kind = uniform(ri.kind);
        u.n = uniform((u.tend - u.t0 + 15) >> 4);
        u.chunks = uniform((u.cols + UC - 1) / UC);
    };

    // ---- locate the range's ends: the row (prefix scans of augmented
    // sub-tile counts), then unit and sub-tile of the first real sub-tile at
    // or after x0, and the index of the first one at or after x1 (T past the
    // end).  `tl` / `un` are the found row's sub-tiles and units.
    struct Found { int row, pre, upre, tl, un; };
    Found f0{}, f1{};
    {
        bool got0 = false, got1 = !has_end;
        auto test = [&](int base, int pre, int upre, int incl, int uincl, int tl, int un) {
            const int64_t ainc = (int64_t)(pre + incl) + (int64_t)C * (upre + uincl);
            auto take = [&](Found &fd, uint64_t hit) {
                const int f = __builtin_ctzll(hit);
                fd.row = base + f;
                fd.pre = pre + __builtin_amdgcn_readlane(incl - tl, f);
                fd.upre = upre + __builtin_amdgcn_readlane(uincl - un, f);
                fd.tl = __builtin_amdgcn_readlane(tl, f);
                fd.un = __builtin_amdgcn_readlane(un, f);
            };
            if (!got0) {
                const uint64_t hit = __builtin_amdgcn_ballot_w64(ainc > x0);
                if (hit) { take(f0, hit); got0 = true; }
            }
            if (!got1) {
                const uint64_t hit = __builtin_amdgcn_ballot_w64(ainc > x1);
                if (hit) { take(f1, hit); got1 = true; }
            }
        };
        if (cached) {
            static_for<0, kCachedBatches>([&]<int b>() {
                if (got0 && got1) return;
                test(b * kWave, 0, 0, inc[b], uinc[b], tlc[b], unc[b]);
            });
        } else {
            int pre = 0, upre = 0;
            for (int base = 0; base < R && !(got0 && got1); base += kWave) {
                const int r = base + lane;
                int tl = 0, un = 0;
                if (r < R) {
                    const RowInfo ri = row_info(r, ld_vec);
                    const int n = tiles_of(ri);
                    un = n > 0 ? Hkv * chunks_of(ri) : 0;
                    tl = un * n;
                }
                const int incl = wave_incl_scan(tl, lane);
                const int uincl = wave_incl_scan(un, lane);
                test(base, pre, upre, incl, uincl, tl, un);
                pre += __builtin_amdgcn_readlane(incl, kWave - 1);
                upre += __builtin_amdgcn_readlane(uincl, kWave - 1);
            }
        }
    }
    // index of the first real sub-tile at or after x in the found row; also
    // its unit (within the row) and sub-tile
    auto settle = [&](int64_t x, const Found &fd, int &uir, int &sub) -> int {
        const int n = uniform(fd.tl / fd.un);
        const int64_t rem = x - ((int64_t)uniform(fd.pre) + (int64_t)C * uniform(fd.upre));
        uir = (int)(rem / (n + C));
        const int o = (int)(rem - (int64_t)uir * (n + C)) - C;
        sub = o > 0 ? o : 0;
        return uniform(fd.pre) + uir * n + sub;
    };
    // Shared mode: a range end that falls inside a unit no longer than the
    // average range moves to the nearer end of that unit (the later one on a
    // tie), so that short units -- a sequence's own suffix -- are never split
    // between waves: every piece of a unit costs a record and a segment.  The
    // ends inside longer units stay where they are, so the closed-form owner
    // of their sub-tiles still holds, and a short unit has one owner.  Two
    // ends that move to the same place leave a wave without work.
    const int64_t nshort = mode == kModeShared ? TA / Weff : 0;
    auto round_end = [&](int g, int n, int sub) -> int {
        if (sub == 0 || n > nshort) return g;
        return 2 * sub < n ? g - sub : g + (n - sub);
    };
    MCursor cur{};
    int g0, sub0, n0;
    {
        cur.row = uniform(f0.row);
        cur.pre = uniform(f0.pre);
        cur.upre = uniform(f0.upre);
        load_row(cur);
        int uir;
        g0 = settle(x0, f0, uir, sub0);
        n0 = cur.n;
        cur.sub = sub0;
        cur.kvh = uir / cur.chunks;
        cur.chunk = uir - cur.kvh * cur.chunks;
    }
    int g1 = T;
    if (has_end) {
        int uir, sub;
        g1 = settle(x1, f1, uir, sub);
        g1 = round_end(g1, uniform(f1.tl / f1.un), sub);
    }
    auto advance = [&](MCursor &u) {
        if (++u.sub < u.n) return;
        u.sub = 0;
        if (++u.chunk < u.chunks) return;
        u.chunk = 0;
        if (++u.kvh < Hkv) return;
        u.kvh = 0;
        u.pre += Hkv * u.chunks * u.n;
        u.upre += Hkv * u.chunks;
        do {
            ++u.row;
            load_row(u);
        } while (u.n == 0 && u.row + 1 < R);
    };
    {
        const int g0r = round_end(g0, n0, sub0);
        if (g0r >= g1) return;
        if (g0r < g0) {
            cur.sub = 0;
        } else if (g0r > g0) {
            // the range starts at the next unit (it exists: g0r < g1 <= T)
            cur.sub = cur.n - 1;
            advance(cur);
        }
        g0 = g0r;
    }
    auto unit_index = [&](const MCursor &u) { return u.upre + u.kvh * u.chunks + u.chunk; };
    auto unit_first = [&](const MCursor &u) { return u.pre + (u.kvh * u.chunks + u.chunk) * u.n; };

    const char *kc = static_cast<const char *>(a.k_cache);
    const char *vc = static_cast<const char *>(a.v_cache);
    const int BS = 1 << a.block_shift;
    const int64_t head_bytes = (int64_t)BS * ROW;
    const int64_t block_bytes = (int64_t)Hkv * head_bytes;
    const int koff = c * ROW + 16 * rg;              // K: token c, bytes 64b + 16rg ..
    const int voff = 4 * rg * ROW + c * DL * EB;     // V: tokens 4rg + m, dims c*DL ..

    auto issue = [&](const MCursor &u, bool live, u32x4 (&kr)[NLK], VReg (&vr)[4]) {
        const int tok = u.t0 + (u.sub << 4);
        const int j = tok >> a.block_shift;
        const int row0 = tok - (j << a.block_shift);
        int rows = u.tend - tok;
        rows = rows < 16 ? rows : 16;
        rows = live ? rows : 0;
        const const_i32_ptr table = (const_i32_ptr)(a.block_tables + (int64_t)u.tseq * a.max_blocks_per_seq);
        const int64_t phys = table[j];
        const int64_t off = uniform(phys * block_bytes + (int64_t)u.kvh * head_bytes + (int64_t)row0 * ROW);
        const int nbytes = uniform(rows * ROW);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(kc + off), 0, nbytes, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)(vc + off), 0, nbytes, kBufferFlags);
        static_for<0, NLK>([&]<int b>() { kr[b] = load_stream(rk, koff + 64 * b); });
        static_for<0, 4>([&]<int m>() {
            if constexpr (VW == 2) {
                const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, voff + m * ROW, 0, kStreamNT));
                vr[m].w[0] = x[0];
                vr[m].w[1] = x[1];
            } else {
                static_for<0, VW / 4>([&]<int h>() {
                    const u32x4 x = load_stream(rv, voff + m * ROW + 16 * h);
                    static_for<0, 4>([&]<int k>() { vr[m].w[4 * h + k] = x[k]; });
                });
            }
        });
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- per-unit state, one set per column chunk ch: lane (rg, c) holds
    // column ch * 16 + c of the unit
    u32x4 qr[CH][NLK];       // B operand of the scores (zero for absent columns)
    int lim[CH];             // the column attends positions [lo, lim)
    int64_t orow[CH];        // multi/suffix: output row of the column; prefix: record index; -1 absent
    float m_run[CH], l_run[CH];   // reference and this lane's share of the exp-sum
    f32x4 acc[CH][DL];       // acc[ch][e][i]: dim (4rg + i) * DL + e
    int nch = CH;            // chunks of the unit with at least one column (wave-uniform)
    int seg_first = g0;

    auto start_unit = [&](const MCursor &u) {
        int64_t qbase = 0;                          // first q row of the row
        int qspan = 0;                              // q rows of the row
        if (u.kind == kRowMulti) {
            qbase = (int64_t)u.row * Tq * Hq;
            qspan = Tq * Hq;
        } else if (u.kind == kRowPrefix) {
            qbase = (int64_t)u.tseq * Hq;
            qspan = (u.cols / G) * Hq;
        } else {
            qbase = (int64_t)u.tseq * Hq;
            qspan = Hq;
        }
        const RowInfo ri{u.t0, u.tend, u.lo, u.L, u.tseq, u.cols, u.kind};
        nch = uniform(min(CH, (u.cols - u.chunk * CH * kMultiCols + kMultiCols - 1) / kMultiCols));
        const char *qb = static_cast<const char *>(a.q) + uniform(qbase * ROW);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)qb, 0, uniform(qspan * ROW), kBufferFlags);
        static_for<0, CH>([&]<int ch>() {
            const int x = (u.chunk * CH + ch) * kMultiCols + c;   // column index within the row
            orow[ch] = column_row(a, u.row, ri, u.kvh, x);
            const bool valid = orow[ch] >= 0;
            if (u.kind == kRowMulti) lim[ch] = valid ? u.L - Tq + x / G + 1 : 0;
            else lim[ch] = valid ? u.L : 0;
            // q rows are the output rows (the prefix records are indexed the same way)
            const int qoff = valid ? (int)(orow[ch] - qbase) * ROW + 16 * rg : 0x7FFFFF00;   // out of range: zero
            static_for<0, NLK>([&]<int b>() { qr[ch][b] = load_chunk(rq, qoff + 64 * b); });
            m_run[ch] = kNegInf;
            l_run[ch] = 0.f;
            static_for<0, DL>([&]<int e>() { acc[ch][e] = f32x4{0.f, 0.f, 0.f, 0.f}; });
        });
        // wait for q here, so that the sub-tile loop is entered with nothing
        // but its own loads in flight and its waits stay exact
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
#pragma unroll
            for (int b = 0; b < NLK; ++b) asm volatile("" ::"v"(qr[ch][b]));
        }
    };

    // One sub-tile: scores, the column-wise online softmax, O^T += V^T P, for
    // every column chunk of the unit (the V operand is packed once).
    auto process = [&](const MCursor &u, const u32x4 (&kr)[NLK], const VReg (&vr)[4]) {
        const int tok = u.t0 + (u.sub << 4) + 4 * rg;
        const int lo = u.lo;
        u32x2 ph[CH], pl[CH];
        float pf[CH][4];   // fp32: the probabilities themselves
        static_for<0, CH>([&]<int ch>() {
            if (ch > 0 && ch >= nch) return;   // a chunk with no column: no work
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            static_for<0, NLK>([&]<int b>() { s = mfma_chunk<DT>(kr[b], qr[ch][b], s); });
            float sv[4];
            float tmax = kNegInf;
            static_for<0, 4>([&]<int r>() {
                const int t = tok + r;
                sv[r] = (t >= lo && t < lim[ch]) ? s[r] * a.scale_log2 : kNegInf;
                tmax = fmaxf(tmax, sv[r]);
            });
            // The exponentials are taken against the column's reference
            // m_run, which is raised (and the state rescaled) only when some
            // score of the wave exceeds its column's reference by more than
            // kLazyRescale (base-2 units).  Weights therefore stay below
            // 2^kLazyRescale, and the common sub-tile needs no exchange
            // between the row groups.  The first valid score of a column
            // always raises its reference.
            if (__builtin_amdgcn_ballot_w64(tmax > m_run[ch] + kLazyRescale) != 0) {
                float cm = fmaxf(tmax, xor16(tmax));
                cm = fmaxf(cm, xor32(cm, lane));
                const float m_new = fmaxf(m_run[ch], cm);
                const float alpha = fast_exp2(m_run[ch] - (m_new == kNegInf ? 0.f : m_new));
                l_run[ch] *= alpha;
                static_for<0, DL>([&]<int e>() { acc[ch][e] *= alpha; });
                m_run[ch] = m_new;
            }
            const float mu = m_run[ch] == kNegInf ? 0.f : m_run[ch];
            float p[4];
            static_for<0, 4>([&]<int r>() { p[r] = fast_exp2(sv[r] - mu); });
            l_run[ch] += (p[0] + p[1]) + (p[2] + p[3]);
            if constexpr (std::is_same_v<DT, BF16>) split_probs_bf16(p, ph[ch], pl[ch]);
            else if constexpr (std::is_same_v<DT, F16>) ph[ch] = pack_probs_f16(p);
            else static_for<0, 4>([&]<int r>() { pf[ch][r] = p[r]; });
        });
        if constexpr (kF32) {
            // 16x16x4 fp32 MFMA, step r over tokens {4k + r}: the B operand of
            // lane (k, j) is its own probability r, the A operand V row 4k + r
            static_for<0, DL>([&]<int e>() {
                static_for<0, 4>([&]<int r>() {
                    const float av = as_f(vr[r].w[e]);
                    static_for<0, CH>([&]<int ch>() {
                        if (ch == 0 || ch < nch)
                            acc[ch][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, pf[ch][r], acc[ch][e], 0, 0, 0);
                    });
                });
            });
        } else {
            static_for<0, DL>([&]<int e>() {
                const u32x2 av = {v_half<e>(vr[0]) | (v_half<e>(vr[1]) << 16),
                                  v_half<e>(vr[2]) | (v_half<e>(vr[3]) << 16)};
                static_for<0, CH>([&]<int ch>() {
                    if (ch == 0 || ch < nch) acc[ch][e] = mfma_pv<DT>(av, ph[ch], acc[ch][e]);
                });
                if constexpr (std::is_same_v<DT, BF16>) {
                    static_for<0, CH>([&]<int ch>() {
                        if (ch == 0 || ch < nch) acc[ch][e] = mfma_pv<DT>(av, pl[ch], acc[ch][e]);
                    });
                }
            });
        }
    };

    // ---- results.  A lane's dims in record / output order: (i, e) -> i * DL + e.
    auto column_sum = [&](float x) {
        x += xor16(x);
        return x + xor32(x, lane);
    };
    // Writes (acc / l) of one column, rounded to the output type.
    auto write_final = [&](int64_t row, const f32x4 (&ac)[DL], float l) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        char *o = static_cast<char *>(a.out) + row * ROW + rg * DQ * EB;
        static_for<0, 4>([&]<int i>() {
            if constexpr (kF32) {
                static_for<0, DL / 4>([&]<int h>() {
                    *reinterpret_cast<f32x4 *>(o + (i * DL + 4 * h) * 4) =
                        f32x4{ac[4 * h][i] * inv, ac[4 * h + 1][i] * inv, ac[4 * h + 2][i] * inv, ac[4 * h + 3][i] * inv};
                });
            } else {
                float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                static_for<0, DL>([&]<int e>() { f[e] = ac[e][i] * inv; });
                const u32x4 pk = pack_chunk<DT>(f);
                if constexpr (DL == 8) *reinterpret_cast<u32x4 *>(o + i * 16) = pk;
                else *reinterpret_cast<u32x2 *>(o + i * 8) = u32x2{pk[0], pk[1]};
            }
        });
    };
    // Stores a (max, exp-sum, acc) record of one column: acc at racc + col * D,
    // (max, sum) at rml + 2 * col.
    auto store_record = [&](float *racc, float *rml, int racc_bytes, int col, float m, float l,
                            const f32x4 (&ac)[DL], bool coherent) {
        static_for<0, 4>([&]<int i>() {
            static_for<0, DL / 4>([&]<int v>() {
                const f32x4 x = {ac[4 * v][i], ac[4 * v + 1][i], ac[4 * v + 2][i], ac[4 * v + 3][i]};
                const int off = (col * D + rg * DQ + i * DL + 4 * v) * 4;
                if (coherent) store_coherent(racc, racc_bytes, off, x);
                else *reinterpret_cast<f32x4 *>(reinterpret_cast<char *>(racc) + off) = x;
            });
        });
        if (rg == 0) {
            if (coherent) {
                __hip_atomic_store(rml + 2 * col, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(rml + 2 * col + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                rml[2 * col] = m;
                rml[2 * col + 1] = l;
            }
        }
    };
    // Stores this segment's record (all chunks) at `slot` of the record array.
    auto store_segment = [&](int64_t slot, const float (&m)[CH], const float (&l)[CH], const f32x4 (&ac)[CH][DL]) {
        float *ra = a.ws_acc + slot * kRecFloats;
        float *rm = a.ws_ml + slot * UC * 2;
        static_for<0, CH>([&]<int ch>() {
            if (orow[ch] >= 0) store_record(ra, rm, 0, ch * kMultiCols + c, m[ch], l[ch], ac[ch], false);
        });
    };
    // The range's first segment, when its unit began in an earlier range and
    // ends inside this one, is held until the end of the range (one column
    // chunk only: two would not fit the registers).
    constexpr bool kHoldFirst = CH == 1;
    float hm[CH], hl[CH];
    f32x4 hacc[CH][DL];
    int64_t hslot = -1;
    // Leaves the unit at `u` after sub-tile `g_last`.
    //  * multi mode: a unit inside this wave's range is finished here; a unit
    //    split between k waves leaves k records (one per wave, at slot
    //    wave + unit), and the wave holding its first sub-tile describes it
    //    (first slot, k, row, KV head, chunk, ...) for the reduce pass;
    //  * shared mode: every unit leaves records (a sequence's result needs its
    //    prefix and its suffix part), and the wave holding the first
    //    sub-tile describes each of the unit's columns for the reduce pass:
    //    where its records start, how many, which column of the records, and
    //    (suffix) whether a prefix part exists.
    auto finish_unit = [&](const MCursor &u, int g_last) {
        float m[CH], l[CH];
        static_for<0, CH>([&]<int ch>() {
            l[ch] = column_sum(l_run[ch]);
            m[ch] = m_run[ch];
        });
        const int ua = unit_first(u);
        const int ub = ua + u.n;
        const int unit = unit_index(u);
        const bool whole = seg_first == ua && g_last + 1 == ub;
        typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
        if (seg_first == ua) {
            // augmented position of the unit's last sub-tile: past the
            // ghosts of every unit up to this one
            const int k = whole ? 1 : wave_of((int64_t)ub - 1 + (int64_t)C * (unit + 1)) - wave + 1;
            if (mode == kModeMulti) {
                if (lane == 0) {
                    int32_t *d = a.unit_desc + kDescWords * (1 + (int64_t)unit);
                    *reinterpret_cast<i32x4 *>(d) = i32x4{wave + unit, k, u.row, (u.kvh << 16) | u.chunk};
                    *reinterpret_cast<i32x4 *>(d + 4) = i32x4{u.tseq, u.cols, u.lo, 0};
                }
            } else if (rg == 0) {
                int32_t *cd = a.col_desc + (u.kind == kRowPrefix ? (int64_t)kColDescWords * a.num_seqs * Hq : 0);
                const int flags = u.kind == kRowSuffix && u.lo > 0 ? kHasPrefix : 0;
                static_for<0, CH>([&]<int ch>() {
                    if (orow[ch] >= 0)
                        *reinterpret_cast<i32x4 *>(cd + kColDescWords * orow[ch]) =
                            i32x4{wave + unit, k, ch * kMultiCols + c, flags};
                });
            }
        }
        if (whole && mode == kModeMulti) {
            static_for<0, CH>([&]<int ch>() {
                if (orow[ch] >= 0) write_final(orow[ch], acc[ch], l[ch]);
            });
            return;
        }
        if constexpr (kHoldFirst) {
            if (seg_first != ua && g_last + 1 < g1) {
                // the range's first segment, of a unit begun in an earlier
                // range, ending inside the range: held in registers and
                // written at the end of the range (a store burst in the
                // middle of the stream holds up the loads queued behind it)
                static_for<0, CH>([&]<int ch>() {
                    hm[ch] = m[ch];
                    hl[ch] = l[ch];
                    static_for<0, DL>([&]<int e>() { hacc[ch][e] = acc[ch][e]; });
                });
                hslot = (int64_t)wave + unit;
                return;
            }
        }
        store_segment((int64_t)wave + unit, m, l, acc);
    };

    // ---- main loop over [g0, g1), one outer iteration per segment, kMDepth
    // sub-tiles in flight (same structure as the single-query kernel)
    u32x4 kbuf[kMDepth][NLK];
    VReg vbuf[kMDepth][4];
    MCursor cp = cur;
    MCursor cl = cur;
    int gl = g0;
    issue(cl, true, kbuf[0], vbuf[0]);
    static_for<1, kMDepth - 1>([&]<int m>() {
        const bool more = gl + 1 < g1;
        if (more) {
            advance(cl);
            ++gl;
        }
        issue(cl, more, kbuf[m], vbuf[m]);
    });
    int g = g0;
    while (true) {
        start_unit(cp);
        seg_first = g;
        int brk = 0;
        bool done = false;
        while (!done) {
            static_for<0, kMDepth>([&]<int i>() {
                if (done) return;
                constexpr int nb = (i + kMDepth - 1) % kMDepth;
                const bool more = gl + 1 < g1;
                if (more) {
                    advance(cl);
                    ++gl;
                }
                issue(cl, more, kbuf[nb], vbuf[nb]);
                process(cp, kbuf[i], vbuf[i]);
                if (cp.sub + 1 == cp.n || g + 1 == g1) {
                    brk = i;
                    done = true;
                    return;
                }
                advance(cp);
                ++g;
            });
        }
        finish_unit(cp, g);
        if (g + 1 >= g1) {
            if constexpr (kHoldFirst) {
                if (hslot >= 0) store_segment(hslot, hm, hl, hacc);
            }
            break;
        }
        advance(cp);
        ++g;
        // the next sub-tiles sit in buffers brk + 1, brk + 2, ... (mod kMDepth):
        // bring them to buffers 0, 1, ...
        if constexpr (kMDepth == 2) {
            if (brk == 0) {
                static_for<0, NLK>([&]<int e>() { kbuf[0][e] = kbuf[1][e]; });
                static_for<0, 4>([&]<int e>() { vbuf[0][e] = vbuf[1][e]; });
            }
        } else {
            static_for<0, kMDepth - 1>([&]<int b>() {
                if (brk == b) {
                    u32x4 tk[kMDepth][NLK];
                    VReg tv[kMDepth][4];
                    static_for<0, kMDepth>([&]<int m>() {
                        static_for<0, NLK>([&]<int e>() { tk[m][e] = kbuf[m][e]; });
                        static_for<0, 4>([&]<int e>() { tv[m][e] = vbuf[m][e]; });
                    });
                    static_for<0, kMDepth - 1>([&]<int m>() {
                        constexpr int from = (b + 1 + m) % kMDepth;
                        static_for<0, NLK>([&]<int e>() { kbuf[m][e] = tk[from][e]; });
                        static_for<0, 4>([&]<int e>() { vbuf[m][e] = tv[from][e]; });
                    });
                }
            });
        }
    }
}

// The reduce pass.  Sixteen threads own one output row, each a slice of
// D / 16 dims; a record is read at one column.  The (max, sum) pairs and the
// acc slices of up to kReduceBatch records are loaded together and folded in
// record order, so an output costs one or two round trips whatever the
// number of records.
constexpr int kReduceThreads = 256;
constexpr int kReduceBatch = 16;
constexpr int kMaxReduceGroups = 2048;

template <int D, int UC>
__device__ __forceinline__ void fold_records(const MultiArgs &a, int64_t base, int k, int col, int d0, float &m,
                                             float &l, f32x4 (&acc)[D / 64]) {
    constexpr int NV = D / 64;   // float4s per thread and record
    constexpr int kRecFloats = UC * D;
    // a descriptor left over from a description that broke its
    // preconditions must not send the loads out of the record array
    if (base < 0 || k < 0 || col < 0 || col >= UC || base + k > (int64_t)kMaxWaves + a.max_units) k = 0;
    for (int r0 = 0; r0 < k; r0 += kReduceBatch) {
        const int nb = min(kReduceBatch, k - r0);
        float mb[kReduceBatch], lb[kReduceBatch];
        f32x4 xb[kReduceBatch][NV];
#pragma unroll
        for (int b = 0; b < kReduceBatch; ++b) {
            if (b < nb) {
                const int64_t slot = base + r0 + b;
                mb[b] = a.ws_ml[(slot * UC + col) * 2];
                lb[b] = a.ws_ml[(slot * UC + col) * 2 + 1];
                const f32x4 *src = reinterpret_cast<const f32x4 *>(a.ws_acc + slot * kRecFloats + col * D + d0);
#pragma unroll
                for (int v = 0; v < NV; ++v) xb[b][v] = src[v];
            }
        }
        float mn = m;
#pragma unroll
        for (int b = 0; b < kReduceBatch; ++b) mn = b < nb ? fmaxf(mn, mb[b]) : mn;
        const float mu = mn == kNegInf ? 0.f : mn;
        const float x = fast_exp2(m - mu);
        l *= x;
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] *= x;
#pragma unroll
        for (int b = 0; b < kReduceBatch; ++b) {
            if (b < nb) {
                const float w = fast_exp2(mb[b] - mu);
                l = __builtin_fmaf(w, lb[b], l);
#pragma unroll
                for (int v = 0; v < NV; ++v) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[v][e] = __builtin_fmaf(w, xb[b][v][e], acc[v][e]);
                }
            }
        }
        m = mn;
    }
}

template <typename DT, int D>
__device__ __forceinline__ void write_row(const MultiArgs &a, int64_t orow, int d0, float l, const f32x4 (&acc)[D / 64]) {
    constexpr int NV = D / 64;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < NV; ++v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[4 * v + e] = acc[v][e] * inv;
    }
    constexpr int EB = DT::kBytes;
    char *o = static_cast<char *>(a.out) + orow * (D * EB) + d0 * EB;
    if constexpr (EB == 4) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
            *reinterpret_cast<f32x4 *>(o + 16 * v) = f32x4{f[4 * v], f[4 * v + 1], f[4 * v + 2], f[4 * v + 3]};
    } else {
        const u32x4 pk = pack_chunk<DT>(f);
        if constexpr (NV == 2) *reinterpret_cast<u32x4 *>(o) = pk;
        else *reinterpret_cast<u32x2 *>(o) = u32x2{pk[0], pk[1]};
    }
}

template <typename DT, int D, int CH>
__global__ __launch_bounds__(kReduceThreads) void attn_multi_reduce(MultiArgs a) {
    constexpr int UC = kMultiCols * CH;
    constexpr int NV = D / 64;
    constexpr int kRowsPerGroup = kReduceThreads / 16;
    const int t = threadIdx.x;
    const int d0 = (t & 15) * (D / 16);
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    if (a.mode == kModeShared) {
        // one output row per (sequence, q head): its suffix records, then its
        // prefix records
        const int64_t items = (int64_t)a.num_seqs * a.num_q_heads;
        for (int64_t item = (int64_t)blockIdx.x * kRowsPerGroup + (t >> 4); item < items;
             item += (int64_t)gridDim.x * kRowsPerGroup) {
            const i32x4 sd = *reinterpret_cast<const i32x4 *>(a.col_desc + kColDescWords * item);
            float m = kNegInf, l = 0.f;
            f32x4 acc[NV];
            for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
            fold_records<D, UC>(a, sd[0], sd[1], sd[2], d0, m, l, acc);
            if (sd[3] & kHasPrefix) {
                const i32x4 pd = *reinterpret_cast<const i32x4 *>(a.col_desc + kColDescWords * (items + item));
                fold_records<D, UC>(a, pd[0], pd[1], pd[2], d0, m, l, acc);
            }
            write_row<DT, D>(a, item, d0, l, acc);
        }
        return;
    }
    // multi mode: the units the main pass split, one per group of 16 rows
    const int units = a.unit_desc[0];
    for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int32_t *d = a.unit_desc + kDescWords * (1 + (int64_t)unit);
        const i32x4 dsc = *reinterpret_cast<const i32x4 *>(d);
        const int k = dsc[1];
        if (k <= 1) continue;
        const i32x4 dsc2 = *reinterpret_cast<const i32x4 *>(d + 4);
        const int row = dsc[2], kvh = dsc[3] >> 16, chunk = dsc[3] & 0xFFFF;
        RowInfo ri{};
        ri.tseq = dsc2[0];
        ri.cols = dsc2[1];
        ri.lo = dsc2[2];
        ri.kind = kRowMulti;
        for (int col = t >> 4; col < UC; col += kRowsPerGroup) {
            const int64_t orow = column_row(a, row, ri, kvh, chunk * UC + col);
            if (orow < 0) continue;
            float m = kNegInf, l = 0.f;
            f32x4 acc[NV];
            for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
            fold_records<D, UC>(a, dsc[0], k, col, d0, m, l, acc);
            write_row<DT, D>(a, orow, d0, l, acc);
        }
    }
}

template <typename DT, int D, int CH>
hipError_t launch_multi_typed(const MultiArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.num_waves / kWavesPerGroup));
    attn_multi_kernel<DT, D, CH><<<grid, dim3(kWavesPerGroup * kWave), 0, stream>>>(a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    // the reduce pass: enough workgroups to cover the split units (multi) or
    // the output rows (shared) in one round
    int64_t groups = a.mode == kModeShared ? ((int64_t)a.num_seqs * a.num_q_heads + 15) / 16 : a.max_units;
    groups = groups < kMaxReduceGroups ? groups : kMaxReduceGroups;
    attn_multi_reduce<DT, D, CH><<<dim3((unsigned)(groups > 0 ? groups : 1)), dim3(kReduceThreads), 0, stream>>>(a);
    return hipGetLastError();
}

template <typename DT, int D, int CH>
int multi_waves_typed() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_multi_kernel<DT, D, CH>, kWavesPerGroup * kWave,
                                                     0) != hipSuccess)
        return 0;
    return blocks * kWavesPerGroup;
}

template <typename DT, int D>
hipError_t launch_multi_chunks(int chunks, const MultiArgs &a, hipStream_t stream) {
    return chunks == 2 ? launch_multi_typed<DT, D, 2>(a, stream) : launch_multi_typed<DT, D, 1>(a, stream);
}
template <typename DT, int D>
int multi_waves_chunks(int chunks) {
    return chunks == 2 ? multi_waves_typed<DT, D, 2>() : multi_waves_typed<DT, D, 1>();
}

}  // namespace

bool multi_supported(int32_t dtype, int32_t head_dim) {
    return (dtype == 0 || dtype == 1 || dtype == 2) && (head_dim == 64 || head_dim == 128);
}

int multi_waves_per_cu(int32_t dtype, int32_t head_dim, int32_t chunks) {
    static std::atomic<int> cache[3][2][kMultiChunksMax];
    if (!multi_supported(dtype, head_dim) || chunks < 1 || chunks > kMultiChunksMax) return 0;
    const int di = dtype, hi = head_dim == 128 ? 1 : 0;
    int v = cache[di][hi][chunks - 1].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (dtype == 0) v = head_dim == 128 ? multi_waves_chunks<F32, 128>(chunks) : multi_waves_chunks<F32, 64>(chunks);
    else if (dtype == 1) v = head_dim == 128 ? multi_waves_chunks<F16, 128>(chunks) : multi_waves_chunks<F16, 64>(chunks);
    else v = head_dim == 128 ? multi_waves_chunks<BF16, 128>(chunks) : multi_waves_chunks<BF16, 64>(chunks);
    if (v > 0) cache[di][hi][chunks - 1].store(v, std::memory_order_relaxed);
    return v;
}

hipError_t launch_attn_multi(int32_t dtype, int32_t head_dim, int32_t chunks, const MultiArgs &a,
                             hipStream_t stream) {
    if (dtype == 0) {
        return head_dim == 128 ? launch_multi_chunks<F32, 128>(chunks, a, stream)
                               : launch_multi_chunks<F32, 64>(chunks, a, stream);
    }
    if (dtype == 1) {
        return head_dim == 128 ? launch_multi_chunks<F16, 128>(chunks, a, stream)
                               : launch_multi_chunks<F16, 64>(chunks, a, stream);
    }
    if (dtype == 2) {
        return head_dim == 128 ? launch_multi_chunks<BF16, 128>(chunks, a, stream)
                               : launch_multi_chunks<BF16, 64>(chunks, a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
