// Paged decode attention for gfx950: one query token per sequence attends over
// a KV cache held in fixed-size physical blocks reached through a Block Table.
//
// What is computed ("PagedAttention核心思想" sections 2.2, 2.3 and 2.5; CSDN
// answer "VLLM中PagedAttention如何降低显存碎片？" section 三 items 4-6 and 9,
// section 四; "PagedAttention技术解析" sections 2.2 and 3.1): for each block of
// the sequence, look its physical id up in the table, score the query against
// the block's keys, fold the scores into a running (max, exp-sum) softmax and
// accumulate the probability-weighted values; tokens past the sequence end in
// the last block are masked out (never loaded, score -inf).  Long sequences
// are cut into pieces whose partial results are merged afterwards (the
// partitioned "V2" scheme the CSDN answer mentions).
//
// Work split (one launch).  A unit is one (sequence, KV head) pair; its work
// is ceil(L/16) sub-tiles of 16 tokens.  All sub-tiles of all units, in
// (sequence, KV head, position) order, are cut into W contiguous ranges, one
// per wave, W being what the GPU holds at once (one wave per SIMD).  The cut
// is even once every unit is charged a few sub-tiles more for the fixed cost
// of starting and finishing it, so every wave takes about the same time
// whatever the length mix, with no empty workgroups and no tail of short
// partitions.  A unit that lies wholly inside one wave's range is finished by
// that wave; a unit shared by k waves gets k partial results (max, exp-sum,
// un-normalised output) in the workspace, and the wave that arrives last at
// the unit's counter merges them in a fixed order and writes the output.  The
// counter is reset to zero by that wave, so the workspace is left as it was
// found.  A wave whose range begins inside a unit keeps that first segment's
// state in registers and writes it as a record only at the end of its range,
// with the last segment's: records are written through to memory, and a
// store in the middle of the stream would hold up every load issued after it.
//
// One wave, one sub-tile (16 tokens of one KV head, the G query heads that
// share it):
//  * K and V rows come in with 16-byte raw buffer loads whose descriptor spans
//    only the sub-tile's valid rows: tail rows of the last block read as zero
//    and are never fetched.  The loads are marked non-temporal (read once).
//    The next sub-tile's loads are issued before the current one is consumed,
//    and the next unit's q before its unit's last sub-tile.
//  * q.K is one 16x16 MFMA product per 32 (bf16/fp16) or 4 (fp32) dims: the
//    16 tokens are the rows, the query heads the columns (up to 16, so any
//    group size fits).  Lane (r, j) receives the scores of tokens 4r..4r+3 of
//    the sub-tile for head j.
//  * Softmax runs as four interleaved streams, one per row group r (tokens
//    4r..4r+3 of every sub-tile), each with its own running max and exp-sum,
//    so a sub-tile needs no exchange between row groups.  The four streams are
//    combined once, when the wave leaves the unit.
//  * The lanes of row group r also hold V rows 4r..4r+3; probabilities and
//    rescale factors reach them by DPP row broadcast, and acc += p V runs on
//    the VALU in fp32.
//  * In a fused step (append + decode) the appended token is the last row of
//    the unit's last sub-tile: its K and V rows are loaded from k_new / v_new
//    into the lanes that hold that row, and those lanes also store it into its
//    slot.  The arithmetic is then the same as a decode after a separate append.
//  * The summation order depends only on logical token positions and on the
//    sizes of the problem, so results are bitwise reproducible and independent
//    of where the blocks live physically or how large the blocks are.
#include "pkv_device.h"

#include <atomic>

namespace pkv {
namespace {

constexpr int kDirectMerge = 8;  // units split in at most this many pieces merge in one level
// Fixed cost of a segment (the lane reductions and the partial record or
// output), in sub-tiles of streaming.  The split charges it to the wave whose
// range holds the start of a unit.
#ifndef PKV_UNIT_COST
#define PKV_UNIT_COST 4
#endif
constexpr int kUnitCost = PKV_UNIT_COST;
#ifndef PKV_DEPTH
#define PKV_DEPTH 2
#endif
// Ablation build only (-DPKV_QK_VALU=1, `python -m paged_kv_cache_353_amd.build
// --qk-valu`): q.K on the VALU instead of the matrix cores, for bf16 at
// head_dim 128 with up to 4 query heads per KV head -- each lane takes dot2
// products over 8 dims of 4 K rows and four DPP steps sum the 16 lanes of a
// row -- so that what MFMA saves can be measured.  The library itself is
// built without it.
#ifndef PKV_QK_VALU
#define PKV_QK_VALU 0
#endif
constexpr int kDepth = PKV_DEPTH;  // sub-tiles in flight per wave

// Position of a wave's load or compute stage in the (sequence, KV head,
// sub-tile) order.  Every field is wave-uniform.
struct Cursor {
    int seq;   // sequence
    int kvh;   // KV head
    int sub;   // sub-tile inside the unit
    int n;     // sub-tiles of the unit
    int L;     // tokens the sequence attends to
    int pre;   // sub-tiles of one KV head summed over the sequences before `seq`
    int cnt;   // sequences before `seq` with at least one sub-tile
};

// ------------------------------------------------------------------ the kernel
// No occupancy is forced on the compiler: the 16-bit, 4-head configuration at
// head_dim 128 runs one wave per SIMD.  Two per SIMD (held to 256 registers)
// measured slower: the older wave of each SIMD takes the memory pipeline and
// the younger one finishes its equal share long after it.
template <typename DT, int D, int G>
__global__ __launch_bounds__(kWavesPerGroup * kWave) void attn_stream_kernel(DecodeArgs a) {
    constexpr int EB = DT::kBytes;
    constexpr int VEC = 16 / EB;          // elements per 16-byte chunk
    constexpr int R = D * EB / 16;        // 16-byte chunks per token row
    constexpr int NL = R / 4;             // 16-byte loads per lane per sub-tile, K and V each
    constexpr int NCH = R >= 16 ? R / 16 : 1;  // distinct V chunks (dims) a lane accumulates
    constexpr int ROW = D * EB;           // bytes per token row
    static_assert(R == 8 || R == 16 || R == 32, "row must be 8, 16 or 32 chunks");
    static_assert(G >= 1 && G <= 16, "query heads per KV head must fit the 16 MFMA columns");

    const int lane = threadIdx.x & (kWave - 1);
    const int rg = lane >> 4;   // row group
    const int c = lane & 15;    // lane inside the row
    const int wave = uniform((int)blockIdx.x * kWavesPerGroup + (int)(threadIdx.x >> 6));
    const int S = a.num_seqs, Hkv = a.num_kv_heads, Hq = a.num_q_heads;
    const int Lmax = a.max_context_len, BS = a.block_size;
    const int W = a.num_waves;
    const const_i32_ptr lens = (const_i32_ptr)a.context_lens;
    auto clampL = [&](int L) { L = L < Lmax ? L : Lmax; return L > 0 ? L : 0; };
    // A fused step appends each sequence's new token at position L - 1: the
    // cache holds positions [0, L - 1) and the token itself comes from
    // k_new / v_new, into the registers of the unit's last sub-tile.
    const bool fused = a.k_new != nullptr;
    const int fused_one = uniform(fused ? 1 : 0);

    // contexts with no token: the output is the empty sum (sequence i is
    // written by wave i % W)
    auto zero_out = [&](int i) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        char *o = static_cast<char *>(a.out) + (int64_t)i * Hq * ROW;
        for (int off = lane * 16; off < Hq * ROW; off += kWave * 16) store_chunk(o, Hq * ROW, off, z);
    };

    // ---- total work and this wave's range.  Sub-tiles are ordered (sequence,
    // KV head, position); a unit is a (sequence, KV head) pair with n >= 1 of
    // them.  In a second, augmented order every unit is preceded by C ghost
    // positions that stand for the fixed cost of a segment.  The augmented
    // order is cut into equal ranges, and a wave processes the real sub-tiles
    // of its range: a wave whose range holds unit starts streams fewer of
    // them.  A batch of at most 64 sequences is read and scanned once, and the
    // scan is kept for locating the range.
    const bool one_batch = S <= kWave;
    int N = 0, NU = 0;   // sub-tiles of one KV head, and sequences with any
    int L0 = 0, n0 = 0, incl0 = 0, cinc0 = 0;
    if (one_batch) {
        L0 = lane < S ? clampL(a.context_lens[lane]) : 0;
        if (wave < S && __builtin_amdgcn_readlane(L0, wave) == 0) zero_out(wave);
        n0 = (L0 + 15) >> 4;
        incl0 = wave_incl_scan(n0, lane);
        cinc0 = wave_incl_scan(n0 > 0 ? 1 : 0, lane);
        N = uniform(__builtin_amdgcn_readlane(incl0, kWave - 1));
        NU = uniform(__builtin_amdgcn_readlane(cinc0, kWave - 1));
    } else {
        for (int base = 0; base < S; base += kWave) {
            const int i = base + lane;
            const int L = i < S ? clampL(a.context_lens[i]) : 0;
            N += (L + 15) >> 4;
            NU += L > 0 ? 1 : 0;
        }
        N = uniform(wave_sum_i(N, lane));
        NU = uniform(wave_sum_i(NU, lane));
        for (int i = wave; i < S; i += W)
            if (clampL(lens[i]) == 0) zero_out(i);
    }
    // sub-tile indices fit in 32 bits (the host rejects larger batches);
    // augmented positions and products with a wave count take 64 bits
    const int T = N * Hkv;
    // Ghosts are used only when every range is longer than C, so that no
    // range holds ghosts alone: then every wave gets at least one sub-tile.
    int C = kUnitCost;
    if (((int64_t)T + (int64_t)C * NU * Hkv) / W < C + 1) C = 0;
    const int64_t TA = (int64_t)T + (int64_t)C * NU * Hkv;   // augmented length
    const int Weff = C > 0 ? W : (T < W ? T : W);             // every wave below Weff gets >= 1 sub-tile
    if (wave >= Weff) return;
    const double inv_weff = 1.0 / (double)Weff, inv_ta = 1.0 / (double)TA;
    const int64_t x0 = floor_div(TA * wave, Weff, inv_weff);      // this wave's augmented range
    const int64_t x1 = floor_div(TA * (wave + 1), Weff, inv_weff);
    // the wave whose range holds augmented position x: the largest w with
    // TA * w / Weff <= x
    auto wave_of = [&](int64_t x) -> int {
        const int64_t w = floor_div((x + 1) * Weff - 1, TA, inv_ta);
        return (int)(w < Weff - 1 ? w : Weff - 1);
    };

    // ---- locate the range's ends: the sequence (prefix scan of the augmented
    // sub-tile counts), KV head and sub-tile of the first real sub-tile at or
    // after x0, and the index of the first one at or after x1 (T past the end)
    Cursor cur{}, endc{};
    const bool has_end = x1 < TA;
    auto pick = [&](Cursor &u, int f, int seq0, int pre, int cnt, int L, int n, int incl, int cinc) {
        u.seq = seq0 + f;
        u.L = __builtin_amdgcn_readlane(L, f);
        u.n = __builtin_amdgcn_readlane(n, f);
        u.pre = pre + __builtin_amdgcn_readlane(incl - n, f);
        u.cnt = cnt + __builtin_amdgcn_readlane(cinc - (n > 0 ? 1 : 0), f);
    };
    if (one_batch) {
        const int64_t ainc = (int64_t)(incl0 + C * cinc0) * Hkv;
        pick(cur, __builtin_ctzll(__builtin_amdgcn_ballot_w64(ainc > x0)), 0, 0, 0, L0, n0, incl0, cinc0);
        if (has_end)
            pick(endc, __builtin_ctzll(__builtin_amdgcn_ballot_w64(ainc > x1)), 0, 0, 0, L0, n0, incl0, cinc0);
    } else {
        int pre = 0, cnt = 0;
        bool found0 = false;
        for (int base = 0; base < S; base += kWave) {
            const int i = base + lane;
            const int L = i < S ? clampL(a.context_lens[i]) : 0;
            const int n = (L + 15) >> 4;
            const int incl = wave_incl_scan(n, lane);
            const int cinc = wave_incl_scan(n > 0 ? 1 : 0, lane);
            const int64_t ainc = ((int64_t)(pre + incl) + (int64_t)C * (cnt + cinc)) * Hkv;
            const uint64_t hit0 = __builtin_amdgcn_ballot_w64(ainc > x0);
            if (!found0 && hit0) {
                pick(cur, __builtin_ctzll(hit0), base, pre, cnt, L, n, incl, cinc);
                found0 = true;
            }
            if (found0) {
                const uint64_t hit1 = __builtin_amdgcn_ballot_w64(ainc > x1);
                if (!has_end) break;
                if (hit1) {
                    pick(endc, __builtin_ctzll(hit1), base, pre, cnt, L, n, incl, cinc);
                    break;
                }
            }
            pre += __builtin_amdgcn_readlane(incl, kWave - 1);
            cnt += __builtin_amdgcn_readlane(cinc, kWave - 1);
        }
    }
    // position inside the sequence: KV head, then sub-tile past the ghosts
    auto settle = [&](int64_t x, Cursor &u) -> int {
        const int64_t rem = x - ((int64_t)u.pre + (int64_t)C * u.cnt) * Hkv;
        u.kvh = (int)((uint32_t)rem / (uint32_t)(u.n + C));   // rem < Hkv * (n + C) < 2^32
        const int o = (int)(rem - (int64_t)u.kvh * (u.n + C)) - C;
        u.sub = o > 0 ? o : 0;
        return Hkv * u.pre + u.kvh * u.n + u.sub;
    };
    const int g0 = settle(x0, cur);
    const int g1 = has_end ? settle(x1, endc) : T;
    auto advance = [&](Cursor &u) __attribute__((always_inline)) {
        if (++u.sub < u.n) return;
        u.sub = 0;
        if (++u.kvh < Hkv) return;
        u.kvh = 0;
        u.pre += u.n;
        ++u.cnt;
        do {
            ++u.seq;
            u.L = clampL(lens[u.seq]);
        } while (u.L == 0);
        u.n = (u.L + 15) >> 4;
    };
    auto unit_of = [&](const Cursor &u) { return u.seq * Hkv + u.kvh; };

    const char *kc = static_cast<const char *>(a.k_cache);
    const char *vc = static_cast<const char *>(a.v_cache);
    const int64_t head_bytes = (int64_t)BS * ROW;
    const int64_t block_bytes = (int64_t)Hkv * head_bytes;
    const int subs_per_block = BS >> 4;
    // per-lane byte offsets inside a sub-tile: K as MFMA rows (token = lane % 16,
    // dims 64b + 16*(lane/16) bytes for load b); V rows 4*rg.. (see NL loads)
    const int koff = c * ROW + 16 * rg;
    const int voff = (4 * rg + (c / R)) * ROW + (c % R) * 16;
    // ablation: K rows loaded like V rows (lane (r, c): row 4r + b, dims 8c..8c+7)
    constexpr bool kQkValu = PKV_QK_VALU && std::is_same_v<DT, BF16> && R == 16 && NL >= G;

    // bytes from a cache's base to the first row of the sub-tile at `u`
    auto tile_offset = [&](const Cursor &u) __attribute__((always_inline)) -> int64_t {
        const int j = u.sub / subs_per_block;
        const const_i32_ptr table = (const_i32_ptr)(a.block_tables + (int64_t)u.seq * a.max_blocks_per_seq);
        const int64_t phys = table[j];
        return uniform(phys * block_bytes + (int64_t)u.kvh * head_bytes + (int64_t)((u.sub << 4) - j * BS) * ROW);
    };
    // the sub-tile at `u` ends the unit and holds the appended token of a fused step
    auto holds_new = [&](const Cursor &u) { return fused && u.sub + 1 == u.n; };

    // Issues the K and V loads of the sub-tile at `u`.  The descriptors span
    // only the cached rows of the sub-tile, so rows past them read as zero.
    // The cached rows, L - fused_one - 16 sub, are never negative: a cursor
    // moved past the range's end is given L = fused_one + 16 sub (`park`), an
    // empty range whose loads return zeros and touch no memory, which keeps
    // the number of loads in flight the same on every step.  (A clamp at zero
    // here would be compiled to a vector med3.)
    auto park = [&](Cursor &u) { u.L = fused_one + (u.sub << 4); };
    auto issue = [&](const Cursor &u, u32x4 (&kr)[NL], u32x4 (&vr)[NL]) __attribute__((always_inline)) {
        const int t0 = u.sub << 4;
        // (The operands are taken through readfirstlane: kept in vector
        // registers under register pressure, they would make this a vector
        // computation whose temporary, a register of the buffer being
        // refilled, costs a wait for every load in flight.)
        int rows = uniform(u.L) - uniform(fused_one) - t0;
        rows = rows < 16 ? rows : 16;
        const int64_t off = tile_offset(u);
        const int nbytes = uniform(rows * ROW);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(kc + off), 0, nbytes, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)(vc + off), 0, nbytes, kBufferFlags);
        static_for<0, NL>([&]<int b>() { kr[b] = load_stream(rk, kQkValu ? voff + 256 * b : koff + 64 * b); });
        static_for<0, NL>([&]<int m>() { vr[m] = load_stream(rv, voff + 256 * m); });
        // keep the compute of the previous sub-tile (and its waits) after these
        // loads, so that they are in flight while it runs
        __builtin_amdgcn_sched_barrier(0);
    };
    // In a fused step the unit's last sub-tile takes the appended token's row
    // from k_new / v_new: every lane loads through a descriptor that covers
    // just that row, at an offset that lands inside it only in the lanes that
    // hold the row (the others read zeros), and the result is OR-ed over the
    // zeros the cache descriptor returned for that row.
    u32x4 knew[NL], vnew[NL];
    // The request is made kNewAhead issues before that of the unit's last
    // sub-tile (the rows come from a small array that is not streamed and take
    // longer to arrive), unless the previous unit's rows are still waiting to
    // be used; then at the issue of the last sub-tile itself.
    constexpr int kNewAhead = NL <= 4 ? 2 : 0;   // (fp32 rows take twice the registers)
    int new_unit = -1;   // the unit whose appended rows sit in (or are on their way to) knew/vnew
    auto issue_new = [&](const Cursor &u) __attribute__((always_inline)) {
        const int rn = u.L - 1 - ((u.n - 1) << 4);   // row of the appended token in the unit's last sub-tile
        const int64_t nb = uniform(((int64_t)u.seq * Hkv + u.kvh) * ROW);
        const __amdgpu_buffer_rsrc_t rkn = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(static_cast<const char *>(a.k_new) + nb), 0, ROW, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rvn = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(static_cast<const char *>(a.v_new) + nb), 0, ROW, kBufferFlags);
        // out-of-range offsets (negative ones wrap to huge) read as zero
        static_for<0, NL>([&]<int b>() {
            knew[b] = load_chunk(rkn, kQkValu ? voff - rn * ROW + 256 * b : koff - rn * ROW + 64 * b);
        });
        static_for<0, NL>([&]<int m>() { vnew[m] = load_chunk(rvn, voff - rn * ROW + 256 * m); });
    };

    // ---- per-unit state
    u32x4 qr[NL];                 // B operand: head = lane % 16 (zero past G)
    u32x4 qn[NL];                 // the next unit's, requested ahead
    int qn_unit = -1;             // unit whose q sits in qn
    float m_run = kNegInf;        // lane (rg, j): running max of stream rg, head j (log2 units)
    float l_run = 0.f;            // its exp-sum
    float acc[G][NCH][VEC];       // lane (rg, c): un-normalised output of stream rg

    auto load_q = [&](const Cursor &u, u32x4 (&qd)[NL]) __attribute__((always_inline)) {
        const char *qb = static_cast<const char *>(a.q) + uniform(((int64_t)u.seq * Hq + (int64_t)u.kvh * G) * ROW);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)qb, 0, G * ROW, kBufferFlags);
        const int qoff = c * ROW + 16 * rg;  // head c (out of range, so zero, for c >= G)
        // (ablation: head b's dims 8c..8c+7 in load b)
        static_for<0, NL>([&]<int b>() { qd[b] = load_chunk(rq, kQkValu ? b * ROW + c * 16 : qoff + 64 * b); });
    };
    auto reset_state = [&]() {
        m_run = kNegInf;
        l_run = 0.f;
        static_for<0, G>([&]<int h>() {
            static_for<0, NCH>([&]<int ch>() { static_for<0, VEC>([&]<int e>() { acc[h][ch][e] = 0.f; }); });
        });
    };

    // Merges the four row-group streams of (m, l, acc).  m and l end up in
    // every lane (head = lane % 16); the acc totals are scattered over the
    // rows: of the lane's G * NCH * VEC accumulators, taken in (head, chunk
    // slot, element) order, row r keeps the totals of the r-th quarter (Q
    // values, in runs of RL consecutive elements of one head's chunk), so
    // that the rows share the stores of the results.
    constexpr int NV = G * NCH * VEC;
    constexpr int Q = NV / 4;
    constexpr int RL = Q < VEC ? Q : VEC;
    constexpr int NRUN = Q / RL;
    static_assert(NV % 4 == 0 && Q % RL == 0, "accumulators split in four quarters of whole runs");
    auto combine_rows = [&](float &m, float &l, const float (&ac)[G][NCH][VEC], float (&tot)[Q]) __attribute__((always_inline)) {
        const float M = rows_max4(m);
        const float Mu = M == kNegInf ? 0.f : M;
        const float sc = fast_exp2(m - Mu);
        const float Ls = rows_sum4(l * sc);
        float v[NV];
        static_for<0, G>([&]<int h>() {
            const float s = row_bcast<h>(sc);
            static_for<0, NCH>([&]<int ch>() {
                static_for<0, VEC>([&]<int e>() { v[(h * NCH + ch) * VEC + e] = ac[h][ch][e] * s; });
            });
        });
        static_for<0, Q>([&]<int q>() {
            float x = rows_scatter_sum4(v[q], v[q + Q], v[q + 2 * Q], v[q + 3 * Q]);
            // 8 chunks a row: lanes c and c + 8 hold the two token halves of one chunk
            if constexpr (R == 8) x += row_ror8(x);
            tot[q] = x;
        });
        m = M;
        l = Ls;
    };

    // Chunk index (within a row) of accumulator chunk slot `ch` of this lane.
    auto chunk_of = [&](int ch) { return R == 32 ? ch * 16 + c : (R == 8 ? (c & 7) : c); };
    // lanes that write their totals (with 8 chunks a row, lanes c and c + 8 hold the same)
    const bool writer = R == 8 ? c < 8 : true;
    // run j of this lane's quarter: head, chunk slot and first element
    struct Run { int h, ch, e0; };
    auto run_of = [&](int j) -> Run {
        const int idx0 = rg * Q + j * RL;
        return Run{idx0 / (NCH * VEC), (idx0 / VEC) % NCH, idx0 % VEC};
    };

    auto write_out = [&](const Cursor &u, const float (&tot)[Q], float l) {
        char *ob = static_cast<char *>(a.out) + ((int64_t)u.seq * Hq + (int64_t)u.kvh * G) * ROW;
        static_for<0, NRUN>([&]<int j>() {
            const Run r = run_of(j);
            // the exp-sum of head r.h sits in lane r.h of every row
            const float L = __builtin_bit_cast(
                float, __builtin_amdgcn_ds_bpermute(((lane & ~15) + r.h) << 2, __builtin_bit_cast(int, l)));
            const float inv = 1.f / L;
            float f[16 / EB] = {};
            static_for<0, RL>([&]<int t>() { f[t] = tot[j * RL + t] * inv; });
            const u32x4 pk = pack_chunk<DT>(f);
            const int off = r.h * ROW + chunk_of(r.ch) * 16 + r.e0 * EB;
            if (writer) {
                if constexpr (RL * EB == 16) store_chunk(ob, G * ROW, off, pk);
                else if constexpr (RL * EB == 8) store_b64(ob, G * ROW, off, pk[0], pk[1]);
                else store_b32(ob, G * ROW, off, pk[0]);
            }
        });
    };

    // ---- partial results: records of (max, exp-sum, acc) per query head.
    // A record holds acc[G][D] (fp32, relative to its max) and (max, exp-sum)[G].
    constexpr int kRecAcc = G * D * 4;   // bytes of a record's acc
    constexpr int NF = G * D / 4;        // float4 chunks of a record's acc
    constexpr int CPL = (NF + kWave - 1) / kWave;  // chunks per lane in the flat layout
    auto reset = [&](int32_t *ctr) {
        if (lane == 0) store_counter(ctr, 0);
    };
    // Merges records [first, first + cnt) of a record array into the flat
    // layout (lane holds float4 chunks lane, lane + 64, ...): returns the
    // per-head max and exp-sum (wave-uniform) and the rescaled acc chunks.
    // The order of every sum is fixed by the record indices.
    auto merge_flat = [&](const float *racc, const float *rml, int64_t first, int cnt,
                          float (&Mh)[G], float (&Lh)[G], f32x4 (&fa)[CPL]) {
        // records whose acc chunks are in flight together (fewer when a record
        // takes more registers per lane)
        constexpr int kBatch = CPL <= 2 ? 8 : 2;
        const int hl = lane % G;   // head of this lane's (record, head) pairs
        auto load_batch = [&](int r0, f32x4 (&xb)[kBatch][CPL], float (&mb)[kBatch][CPL]) {
            static_for<0, kBatch>([&]<int b>() {
                const int64_t rr = first + (r0 + b < cnt ? r0 + b : cnt - 1);
                static_for<0, CPL>([&]<int j>() {
                    const int q = j * kWave + lane;
                    const int qc = q < NF ? q : NF - 1;
                    xb[b][j] = load_coherent(racc + rr * G * D, kRecAcc, qc * 16);
                    mb[b][j] = __hip_atomic_load(rml + rr * G * 2 + 2 * ((qc * 4) / D), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                });
            });
        };
        // the first pair of this lane and the first batch of acc chunks are
        // requested together, so the common case costs one round trip
        float m0 = kNegInf, l0 = 0.f;
        if (lane < cnt * G) {
            const int64_t rr = first + lane / G;
            m0 = __hip_atomic_load(rml + rr * G * 2 + 2 * hl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            l0 = __hip_atomic_load(rml + rr * G * 2 + 2 * hl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        f32x4 xb[kBatch][CPL];
        float mb[kBatch][CPL];
        load_batch(0, xb, mb);
        // per-head max and exp-sum over the records: online over this lane's
        // pairs, then a fixed butterfly over the lanes of the same head
        auto fold = [](float &m, float &l, float m2, float l2) {
            const float mn = fmaxf(m, m2);
            const float mu = mn == kNegInf ? 0.f : mn;
            l = l * fast_exp2(m - mu) + l2 * fast_exp2(m2 - mu);
            m = mn;
        };
        float mx = m0, ls = l0;
        for (int pidx = lane + kWave; pidx < cnt * G; pidx += kWave) {
            const int64_t rr = first + pidx / G;
            const float Mr = __hip_atomic_load(rml + rr * G * 2 + 2 * hl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float Lr = __hip_atomic_load(rml + rr * G * 2 + 2 * hl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            fold(mx, ls, Mr, Lr);
        }
        for (int d = G; d < kWave; d <<= 1) {
            const float m2 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ d) << 2, __builtin_bit_cast(int, mx)));
            const float l2 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ d) << 2, __builtin_bit_cast(int, ls)));
            fold(mx, ls, m2, l2);
        }
        const float mu = mx == kNegInf ? 0.f : mx;
        static_for<0, G>([&]<int h>() {
            Mh[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mu), h));
            Lh[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls), h));
        });
        float Mq[CPL];   // max of the head each of this lane's chunks belongs to
        static_for<0, CPL>([&]<int j>() {
            const int hq = ((j * kWave + lane) * 4) / D;
            float v = 0.f;
            static_for<0, G>([&]<int h>() { v = hq == h ? Mh[h] : v; });
            Mq[j] = v;
            fa[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        });
        // weighted sum of the acc chunks, in record order
        for (int r0 = 0; r0 < cnt; r0 += kBatch) {
            if (r0 > 0) load_batch(r0, xb, mb);
            static_for<0, kBatch>([&]<int b>() {
                if (r0 + b < cnt) {
                    static_for<0, CPL>([&]<int j>() {
                        const float w = fast_exp2(mb[b][j] - Mq[j]);
                        static_for<0, 4>([&]<int e>() { fa[j][e] = __builtin_fmaf(w, xb[b][j][e], fa[j][e]); });
                    });
                }
            });
        }
    };
    // Writes a merged result in the flat layout as a record (next tree level).
    auto store_flat_record = [&](float *racc, float *rml, int64_t slot, const float (&Mh)[G],
                                 const float (&Lh)[G], const f32x4 (&fa)[CPL]) {
        static_for<0, CPL>([&]<int j>() {
            const int q = j * kWave + lane;
            if (q < NF) store_coherent(racc + slot * G * D, kRecAcc, q * 16, fa[j]);
        });
        static_for<0, G>([&]<int h>() {
            if (lane == 0) {
                store_coherent_f32(rml + slot * G * 2, G * 8, 8 * h, Mh[h]);
                store_coherent_f32(rml + slot * G * 2, G * 8, 8 * h + 4, Lh[h]);
            }
        });
    };
    // Writes a merged result in the flat layout as the unit's output.
    // Writes a merged result in the flat layout as the output of `unit`
    // (its G query heads are rows unit * G .. unit * G + G - 1 of the output).
    auto write_out_flat = [&](int unit, const float (&Lh)[G], const f32x4 (&fa)[CPL]) {
        char *ob = static_cast<char *>(a.out) + (int64_t)unit * G * ROW;
        static_for<0, CPL>([&]<int j>() {
            const int q = j * kWave + lane;
            if (q < NF) {
                const int hq = (q * 4) / D;
                float lq = 1.f;
                static_for<0, G>([&]<int h>() { lq = hq == h ? Lh[h] : lq; });
                const float inv = 1.f / lq;
                float f[4];
                static_for<0, 4>([&]<int e>() { f[e] = fa[j][e] * inv; });
                if constexpr (EB == 4) {
                    *reinterpret_cast<f32x4 *>(ob + q * 16) = f32x4{f[0], f[1], f[2], f[3]};
                } else {
                    float f8[8] = {f[0], f[1], f[2], f[3], 0.f, 0.f, 0.f, 0.f};
                    const u32x4 pk = pack_chunk<DT>(f8);
                    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                    *reinterpret_cast<u32x2 *>(ob + q * 8) = u32x2{pk[0], pk[1]};
                }
            }
        });
    };

    // ---- a unit shared by k waves leaves k partial records, merged in a
    // two-level tree: groups of about sqrt(k) consecutive segments are merged
    // by the last of their waves to arrive, then the group results by the last
    // group to arrive, so that no wave reads more than about sqrt(k) records
    // (k is known statically from the split).  The record slots of a unit are
    // base .. base + k - 1 with base = w_first + unit.
    struct Split {
        int unit;     // (sequence, KV head) index
        int k;        // waves that share the unit
        int wfirst;   // the first of them
    };
    struct Tree {
        int f1, ng, j, kj;   // group size, groups, this wave's group and its size
    };
    auto split_of = [&](const Cursor &u) -> Split {
        // augmented position of the unit's first sub-tile, past its ghosts
        const int64_t xa = ((int64_t)u.pre + (int64_t)C * u.cnt) * Hkv + (int64_t)u.kvh * (u.n + C) + C;
        Split s;
        s.wfirst = wave_of(xa);
        s.k = wave_of(xa + u.n - 1) - s.wfirst + 1;
        s.unit = unit_of(u);
        return s;
    };
    auto tree_of = [&](const Split &s) -> Tree {
        Tree tr;
        int f1 = (int)__builtin_sqrtf((float)s.k);
        while (f1 * f1 < s.k) ++f1;
        tr.f1 = f1;
        tr.ng = (s.k + f1 - 1) / f1;
        tr.j = (wave - s.wfirst) / f1;
        tr.kj = min(f1, s.k - tr.j * f1);
        return tr;
    };
    // this segment's record
    auto store_record = [&](const Split &s, const float (&sa)[Q], float sm, float sl) __attribute__((always_inline)) {
        const int64_t slot = (int64_t)wave + s.unit;
        float *pacc = a.ws_acc + slot * G * D;
        float *pml = a.ws_ml + slot * G * 2;
        static_for<0, NRUN>([&]<int j>() {
            const Run r = run_of(j);
            const int off = (r.h * D + chunk_of(r.ch) * VEC + r.e0) * 4;
            if (writer) {
                if constexpr (RL >= 4) {
                    static_for<0, RL / 4>([&]<int k>() {
                        const f32x4 x = {sa[j * RL + 4 * k], sa[j * RL + 4 * k + 1], sa[j * RL + 4 * k + 2],
                                         sa[j * RL + 4 * k + 3]};
                        store_coherent(pacc, kRecAcc, off + 16 * k, x);
                    });
                } else {
                    static_for<0, RL>([&]<int k>() { store_coherent_f32(pacc, kRecAcc, off + 4 * k, sa[j * RL + k]); });
                }
            }
        });
        if (rg == 0 && c < G) {
            store_coherent_f32(pml, G * 8, 8 * c, sm);
            store_coherent_f32(pml, G * 8, 8 * c + 4, sl);
        }
    };
    // The arrival of a segment: a relaxed agent-scope add on the unit's (or
    // its group's) counter, issued only once the segment's record stores have
    // completed.  The returned count (in lane 0) is read later.
    auto post_arrival = [&](const Split &s) -> int {
        int32_t *ctr = a.ws_cnt + s.unit;
        if (s.k > kDirectMerge) ctr = a.ws_gcnt + ((int64_t)s.wfirst + s.unit + tree_of(s).j);
        int old = 0;
        if (lane == 0) old = atomic_add_counter(ctr, 1);
        return old;
    };
    // After the arrival returned the count `got`: merges and writes the
    // output if this wave was the last of the unit (or of its group, then of
    // the groups).
    auto complete = [&](const Split &s, int got) {
        float Mh[G], Lh[G];
        f32x4 fa[CPL];
        const int64_t base = (int64_t)s.wfirst + s.unit;
        if (s.k <= kDirectMerge) {
            if (got != s.k - 1) return;
            merge_flat(a.ws_acc, a.ws_ml, base, s.k, Mh, Lh, fa);
            write_out_flat(s.unit, Lh, fa);
            reset(a.ws_cnt + s.unit);
            return;
        }
        const Tree tr = tree_of(s);
        if (got != tr.kj - 1) return;
        const int64_t gslot = base + tr.j;
        merge_flat(a.ws_acc, a.ws_ml, base + (int64_t)tr.j * tr.f1, tr.kj, Mh, Lh, fa);
        store_flat_record(a.ws_gacc, a.ws_gml, gslot, Mh, Lh, fa);
        reset(a.ws_gcnt + gslot);
        wait_vmem_done();
        int og = 0;
        if (lane == 0) og = atomic_add_counter(a.ws_cnt + s.unit, 1);
        if (__builtin_amdgcn_readlane(og, 0) != tr.ng - 1) return;
        merge_flat(a.ws_gacc, a.ws_gml, base, tr.ng, Mh, Lh, fa);
        write_out_flat(s.unit, Lh, fa);
        reset(a.ws_cnt + s.unit);
    };

    // One sub-tile: scores on MFMA, four-stream online softmax, acc += p V.
    auto process_rows = [&](int nvalid, const u32x4 (&kr)[NL], const u32x4 (&vr)[NL]) __attribute__((always_inline)) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kQkValu) {
            typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
            auto bf2 = [](uint32_t u) __attribute__((always_inline)) { return __builtin_bit_cast(bf16x2v, u); };
            float part[4][G];
            static_for<0, 4>([&]<int r>() {
                static_for<0, G>([&]<int h>() {
                    float x = 0.f;
                    static_for<0, 4>([&]<int i>() {
                        const uint32_t ku = kr[r][i], qu = qr[h][i];
                        x = __builtin_amdgcn_fdot2_f32_bf16(bf2(ku), bf2(qu), x, false);
                    });
                    // sum over the 16 lanes of the row: row_ror 8, row_ror 4, quad swaps
                    x += as_f(__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0x128, 0xF, 0xF, false));
                    x += as_f(__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0x124, 0xF, 0xF, false));
                    x += as_f(__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0x4E, 0xF, 0xF, false));
                    x += as_f(__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0xB1, 0xF, 0xF, false));
                    part[r][h] = x;
                });
            });
            // lane (r, c) keeps the score of token 4r + j for head c, as the MFMA leaves it
            static_for<0, 4>([&]<int j>() {
                float v = 0.f;
                static_for<0, G>([&]<int h>() { v = c == h ? part[j][h] : v; });
                s[j] = v;
            });
        } else {
            static_for<0, NL>([&]<int b>() { s = mfma_chunk<DT>(kr[b], qr[b], s); });
        }
        float sv[4];
        float tmax = kNegInf;
        static_for<0, 4>([&]<int r>() {
            sv[r] = (4 * rg + r < nvalid) ? s[r] * a.scale_log2 : kNegInf;
            tmax = fmaxf(tmax, sv[r]);
        });
        const float m_new = fmaxf(m_run, tmax);
        const float mu = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - mu);
        float p[4];
        static_for<0, 4>([&]<int r>() { p[r] = fast_exp2(sv[r] - mu); });
        l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(c < G && alpha != 1.f) != 0) {
            static_for<0, G>([&]<int h>() {
                const float ah = row_bcast<h>(alpha);
                static_for<0, NCH>([&]<int ch>() { static_for<0, VEC>([&]<int e>() { acc[h][ch][e] *= ah; }); });
            });
        }
        // V slot mm of this lane holds token 4*rg + mm (16 chunks a row),
        // mm/2 (32 chunks) or 2*mm + (c >= 8) (8 chunks)
        static_for<0, NL>([&]<int mm>() {
            float vf[VEC];
            chunk_to_f32<DT>(vr[mm], vf);
            constexpr int ch = NCH == 2 ? (mm & 1) : 0;
            static_for<0, G>([&]<int h>() {
                float ph;
                if constexpr (R == 16) ph = row_bcast<h>(p[mm]);
                else if constexpr (R == 32) ph = row_bcast<h>(p[mm >> 1]);
                else ph = row_bcast_split<h>(p[2 * mm], p[2 * mm + 1]);
                static_for<0, VEC>([&]<int e>() { acc[h][ch][e] = __builtin_fmaf(ph, vf[e], acc[h][ch][e]); });
            });
        });
    };
    // The sub-tile at `u`; in a fused step the unit's last one also stores
    // the appended token into its slot, from the lanes that hold its row.
    auto process = [&](const Cursor &u, const u32x4 (&kr)[NL], const u32x4 (&vr)[NL]) __attribute__((always_inline)) {
        if (!holds_new(u)) {
            process_rows(u.L - (u.sub << 4), kr, vr);  // valid rows: >= 1
            return;
        }
        new_unit = -1;   // knew / vnew are taken over below
        u32x4 k2[NL], v2[NL];
        static_for<0, NL>([&]<int b>() { k2[b] = kr[b] | knew[b]; v2[b] = vr[b] | vnew[b]; });
        process_rows(u.L - (u.sub << 4), k2, v2);
        const int rn = u.L - 1 - (u.sub << 4);
        const int64_t so = tile_offset(u) + (int64_t)rn * ROW;
        char *kd = static_cast<char *>(a.k_cache_w) + so;
        char *vd = static_cast<char *>(a.v_cache_w) + so;
        static_for<0, NL>([&]<int b>() {
            if constexpr (kQkValu) {
                const int o = voff + 256 * b;
                if (o / ROW == rn) store_chunk(kd, ROW, o - rn * ROW, knew[b]);
            } else {
                if (c == rn) store_chunk(kd, ROW, 16 * rg + 64 * b, knew[b]);
            }
        });
        static_for<0, NL>([&]<int m>() {
            const int o = voff + 256 * m;
            if (o / ROW == rn) store_chunk(vd, ROW, o - rn * ROW, vnew[m]);
        });
    };
    // Requests the q of the unit after the one `u` ends, when `u` (sub-tile
    // gidx) is its unit's last, that unit lies in this range and no earlier
    // request is still waiting to be taken over.
    auto prefetch_q = [&](const Cursor &u, int gidx) __attribute__((always_inline)) {
        if (u.sub + 1 == u.n && gidx + 1 < g1 && qn_unit < 0) {
            Cursor nx = u;
            advance(nx);
            load_q(nx, qn);
            qn_unit = unit_of(nx);
        }
    };
    // Loads that depend on what the sub-tile just issued at `u` is: the
    // appended token's row and the next unit's q.  They are issued after the
    // step's compute rather than with the sub-tile's loads, so that the wait of
    // that compute (whose count the compiler takes over both paths) does not
    // include them.
    auto issue_extras = [&](const Cursor &u, int gidx) __attribute__((always_inline)) {
        if (fused && u.sub + 1 + kNewAhead >= u.n && new_unit < 0) {
            issue_new(u);
            new_unit = unit_of(u);
        }
        prefetch_q(u, gidx);
    };

    // ---- main loop over [g0, g1), kDepth sub-tiles in flight: each step
    // issues the loads of sub-tile gl + 1 and then consumes sub-tile g,
    // unconditionally (empty ranges past the end), so its waits only ever
    // cover the sub-tile being consumed.  The step is unrolled kDepth times so
    // that the buffers rotate without moves.  A segment (the part of a unit
    // inside the range) that ends before the range does is finished in the
    // loop: a whole unit writes its output; the range's first segment, when
    // its unit began in an earlier range, is set aside (its combined state
    // held in registers).  After the loop the range's last segment and the
    // set-aside one are written as records, their arrivals posted, and any
    // merge this wave owes done.
    u32x4 kbuf[kDepth][NL], vbuf[kDepth][NL];
    Cursor cp = cur;   // the sub-tile being consumed (g)
    Cursor cl = cur;   // the most recently issued sub-tile ...
    int gl = g0;       // ... and its index
    load_q(cur, qr);
    issue(cl, kbuf[0], vbuf[0]);
    issue_extras(cl, gl);
    static_for<1, kDepth - 1>([&]<int m>() {
        const bool more = gl + 1 < g1;
        if (more) {
            advance(cl);
            ++gl;
        } else {
            park(cl);
        }
        issue(cl, kbuf[m], vbuf[m]);
        if (more) issue_extras(cl, gl);
    });
    reset_state();
    int g = g0;
    int seg_first = g0;
    // the split of the current unit, when a record of it may be needed (the
    // range's first unit, and a later one that runs past the range's end):
    // worked out while loads are in flight rather than when the record is due
    Split usplit = split_of(cur);
    bool pend = false;      // the range's first segment ends inside the range (unit begun earlier)
    Split psplit{};
    float hacc[Q];             // its state (this lane's quarter), stored as a record at the end of the range
    float hm = 0.f, hl = 0.f;
    // One step; returns true once sub-tile g1 - 1 has been consumed.  (The loop
    // leaves from the step that ends it, so that its back edge follows a full
    // round of steps, where every buffer's loads have been consumed: the
    // compiler's wait analysis then sees no load in flight into a buffer being
    // refilled.)
    auto step = [&]<int i>() __attribute__((always_inline)) -> bool {
        constexpr int nb = (i + kDepth - 1) % kDepth;
        const bool more = gl + 1 < g1;
        if (more) {
            advance(cl);
            ++gl;
        } else {
            park(cl);   // past the range's end: an empty load range
        }
        issue(cl, kbuf[nb], vbuf[nb]);
        process(cp, kbuf[i], vbuf[i]);
        if (g + 1 == g1) return true;
        if (cp.sub + 1 == cp.n) {
            // a segment ends inside the range
            float tot[Q];
            combine_rows(m_run, l_run, acc, tot);
            const int ua = Hkv * cp.pre + cp.kvh * cp.n;
            if (seg_first == ua) {
                write_out(cp, tot, l_run);
            } else {
                // the range's first segment, of a unit begun in an earlier
                // range: its state is held to the end of the range
                psplit = usplit;
                static_for<0, Q>([&]<int q>() { hacc[q] = tot[q]; });
                hm = m_run;
                hl = l_run;
                pend = true;
            }
            advance(cp);
            ++g;
            seg_first = g;
            if (g + cp.n > g1) usplit = split_of(cp);   // the range's last segment, partial
            if (qn_unit == unit_of(cp)) {
                static_for<0, NL>([&]<int b>() { qr[b] = qn[b]; });
                qn_unit = -1;
            } else {
                // not requested ahead (a unit of one sub-tile before it):
                // wait here, so that no path reaches the next step with q
                // loads in flight and every step's waits stay exact
                load_q(cp, qr);
                wait_vmem_done();
            }
            reset_state();
        } else {
            advance(cp);
            ++g;
        }
        if (more) issue_extras(cl, gl);
        return false;
    };
    while (!static_any<0, kDepth>(step)) {}

    // ---- the range's last segment (sub-tile g1 - 1 was the last consumed)
    float tot[Q];
    combine_rows(m_run, l_run, acc, tot);
    const int ua_last = Hkv * cp.pre + cp.kvh * cp.n;
    const bool last_whole = seg_first == ua_last && g + 1 == ua_last + cp.n;
    Split lsplit{};
    if (last_whole) {
        write_out(cp, tot, l_run);
    } else {
        lsplit = usplit;
        store_record(lsplit, tot, m_run, l_run);
    }
    if (pend) store_record(psplit, hacc, hm, hl);
    if (last_whole && !pend) return;
    wait_vmem_done();   // the records' stores are complete
    int last_old = 0, pend_old = 0;
    if (!last_whole) last_old = post_arrival(lsplit);
    if (pend) pend_old = post_arrival(psplit);
    if (!last_whole) complete(lsplit, __builtin_amdgcn_readlane(last_old, 0));
    if (pend) complete(psplit, __builtin_amdgcn_readlane(pend_old, 0));
}

template <typename DT, int D, int G>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.num_waves / kWavesPerGroup));
    attn_stream_kernel<DT, D, G><<<grid, dim3(kWavesPerGroup * kWave), kDecodeLdsPin, stream>>>(a);
    return hipGetLastError();
}

template <typename DT, int D, int G>
int waves_per_cu_typed() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_stream_kernel<DT, D, G>,
                                                     kWavesPerGroup * kWave, kDecodeLdsPin) != hipSuccess)
        return 0;
    return blocks * kWavesPerGroup;
}

template <typename DT, int D>
hipError_t launch_group(int group, const DecodeArgs &a, hipStream_t s) {
    switch (group) {
        case 1: return launch_typed<DT, D, 1>(a, s);
        case 2: return launch_typed<DT, D, 2>(a, s);
        case 4: return launch_typed<DT, D, 4>(a, s);
        case 8: return launch_typed<DT, D, 8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename DT, int D, int G>
int scratch_typed() {
    hipFuncAttributes attr{};
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(attn_stream_kernel<DT, D, G>)) != hipSuccess)
        return 0;
    return (int)attr.localSizeBytes;
}

template <typename DT, int D>
int scratch_group(int group) {
    switch (group) {
        case 1: return scratch_typed<DT, D, 1>();
        case 2: return scratch_typed<DT, D, 2>();
        case 4: return scratch_typed<DT, D, 4>();
        case 8: return scratch_typed<DT, D, 8>();
        default: return 0;
    }
}

template <typename DT, int D>
int waves_group(int group) {
    switch (group) {
        case 1: return waves_per_cu_typed<DT, D, 1>();
        case 2: return waves_per_cu_typed<DT, D, 2>();
        case 4: return waves_per_cu_typed<DT, D, 4>();
        case 8: return waves_per_cu_typed<DT, D, 8>();
        default: return 0;
    }
}

template <typename DT>
hipError_t launch_dim(int head_dim, int group, const DecodeArgs &a, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_group<DT, 64>(group, a, s);
        case 128: return launch_group<DT, 128>(group, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename DT>
int waves_dim(int head_dim, int group) {
    switch (head_dim) {
        case 64: return waves_group<DT, 64>(group);
        case 128: return waves_group<DT, 128>(group);
        default: return 0;
    }
}

// The scratch of the decode step that allocates nothing: a file-scope device
// array, one copy per GPU, held until the process ends.  Host code uses the
// address hipGetSymbolAddress gives for the current device, never the
// array's name (on the host that names a stand-in, not device memory).
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t *p, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

void *static_scratch(int device, hipStream_t stream) {
    constexpr int kMaxDev = 64;
    static std::atomic<void *> ptrs[kMaxDev];
    if (device < 0 || device >= kMaxDev) return nullptr;
    void *p = ptrs[device].load(std::memory_order_acquire);
    if (p) return p;
    // first use on this device (the caller made it current): look the array
    // up and clear its counter region; later calls leave the counters at zero
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return nullptr;
    if (hipGetSymbolAddress((void **)&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    zero_fill_kernel<<<64, 256, 0, stream>>>(static_cast<uint32_t *>(p), (int64_t)(kStaticCounterBytes / 4));
    if (hipGetLastError() != hipSuccess) return nullptr;
    ptrs[device].store(p, std::memory_order_release);
    return p;
}

bool decode_supported(int32_t dtype, int32_t head_dim, int32_t group) {
    const bool dt = dtype == 0 || dtype == 1 || dtype == 2;
    const bool hd = head_dim == 64 || head_dim == 128;
    const bool gr = group == 1 || group == 2 || group == 4 || group == 8;
    return dt && hd && gr;
}

int decode_waves_per_cu(int32_t dtype, int32_t head_dim, int32_t group) {
    // The occupancy query is slow next to a launch, and its answer is a
    // property of the compiled kernel: ask once per configuration (a racing
    // first call computes the same value twice, which is harmless).
    static std::atomic<int> cache[3][2][4];
    const int hd = head_dim == 128 ? 1 : 0;
    const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : 3;
    if (dtype < 0 || dtype > 2) return 0;
    int v = cache[dtype][hd][gi].load(std::memory_order_relaxed);
    if (v > 0) return v;
    switch (dtype) {
        case 0: v = waves_dim<F32>(head_dim, group); break;
        case 1: v = waves_dim<F16>(head_dim, group); break;
        default: v = waves_dim<BF16>(head_dim, group); break;
    }
    if (v > 0) cache[dtype][hd][gi].store(v, std::memory_order_relaxed);
    return v;
}

int decode_scratch_bytes(int32_t dtype, int32_t head_dim, int32_t group) {
    // a property of the compiled kernel: asked once per configuration
    static std::atomic<int> cache[3][2][4];
    if (!decode_supported(dtype, head_dim, group)) return 0;
    const int hd = head_dim == 128 ? 1 : 0;
    const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : 3;
    int v = cache[dtype][hd][gi].load(std::memory_order_relaxed);
    if (v != 0) return v > 0 ? v : 0;
    int b = 0;
    switch (dtype) {
        case 0: b = head_dim == 128 ? scratch_group<F32, 128>(group) : scratch_group<F32, 64>(group); break;
        case 1: b = head_dim == 128 ? scratch_group<F16, 128>(group) : scratch_group<F16, 64>(group); break;
        default: b = head_dim == 128 ? scratch_group<BF16, 128>(group) : scratch_group<BF16, 64>(group); break;
    }
    cache[dtype][hd][gi].store(b > 0 ? b : -1, std::memory_order_relaxed);
    return b;
}

hipError_t launch_attn_decode(int32_t dtype, int32_t head_dim, int32_t group,
                              const DecodeArgs &a, hipStream_t stream) {
    switch (dtype) {
        case 0: return launch_dim<F32>(head_dim, group, a, stream);
        case 1: return launch_dim<F16>(head_dim, group, a, stream);
        case 2: return launch_dim<BF16>(head_dim, group, a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
