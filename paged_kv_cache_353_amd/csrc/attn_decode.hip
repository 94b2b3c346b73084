// Paged decode attention for gfx950: one query token per sequence attends over
// a KV cache held in fixed-size physical blocks reached through a Block Table.
//
// What is computed ("PagedAttention核心思想" sections 2.2, 2.3 and 2.5; CSDN
// answer "VLLM中PagedAttention如何降低显存碎片？" section 三 items 4-6 and 9,
// section 四; "PagedAttention技术解析" sections 2.2 and 3.1): for each block of
// the sequence, look its physical id up in the table, score the query against
// the block's keys, fold the scores into a running (max, exp-sum) softmax and
// accumulate the probability-weighted values; tokens past the sequence end in
// the last block are masked out (never loaded, score -inf).  Long sequences are
// cut into partitions whose partial results are merged by a second kernel (the
// partitioned "V2" scheme the CSDN answer mentions).
//
// Mapping to CDNA4:
//  * Workgroup = (partition, kv head, sequence), `NW` wave64s.  All G = Hq/Hkv
//    query heads that share the KV head are served by one load of each K/V
//    tile (GQA grouping).
//  * A wave scores 16 tokens at a time.  The (block, kv head) tile of 16 rows
//    is contiguous in HBM; each lane loads 16-byte chunks with raw buffer
//    loads whose descriptor spans only the valid rows, so tail rows of the
//    last block are never fetched (the hardware returns 0 past num_records).
//    Each wave load instruction reads 1 KiB of consecutive bytes.
//  * q.k partials use v_dot2 (bf16/fp16) or FMA (fp32) on the lane's chunk,
//    then a lane reduce-scatter over the R lanes of a row through DPP
//    (mirror / half-mirror / quad permutes), leaving every (token, head) score
//    fully summed in one lane.
//  * Softmax bookkeeping runs in a "one score per lane" layout (head = lane %
//    G); probabilities go through a 256-byte LDS slot per wave to the lanes
//    that hold the matching V chunks; acc[G][8] fp32 per lane.
//  * K/V tiles of the next sub-tile are loaded before the current one is
//    consumed (two register buffers), keeping ~16 KiB in flight per wave.
//  * The summation order depends only on logical token positions, so results
//    are bitwise reproducible and independent of where blocks live physically.
#include "pkv_internal.h"

#include <type_traits>

namespace pkv {
namespace {

constexpr int kWave = 64;
constexpr uint32_t kBufferFlags = 0x00020000u;  // gfx9 buffer descriptor word 3 (32-bit data)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Block Table and length reads go through the constant address space so they
// become scalar loads: a vector load here would make the compiler wait for
// every tile load already in flight (vmcnt is in order) and would turn the
// buffer descriptor into a per-lane value.
typedef const int32_t __attribute__((address_space(4))) *const_i32_ptr;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct F32 { static constexpr int kBytes = 4; };
struct F16 { static constexpr int kBytes = 2; };
struct BF16 { static constexpr int kBytes = 2; };

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f.template operator()<I>();
        static_for<I + 1, N>(f);
    }
}

// Element reinterpretation goes through by-value helpers: hipcc (clang 22)
// miscompiles __builtin_bit_cast applied directly to an ext-vector element
// (it reads element 0 whatever the index).
__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ bf16x2 as_bf2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }
__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// ------------------------------------------------------------------ lane exchange
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kRowMirror = 0x140;   // lane c <-> 15-c within 16
constexpr int kRowHalfMirror = 0x141;  // lane c <-> 7-c within 8

__device__ __forceinline__ float swap16(float x) {  // lane ^ 16 (within 32)
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
__device__ __forceinline__ float swap32(float x, int lane) {  // lane ^ 32
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, x)));
}

// Value from a partner lane whose index differs in bit BIT (and possibly in
// lower bits, which the callers treat as still unreduced).
template <int BIT>
__device__ __forceinline__ float partner(float x, int lane) {
    if constexpr (BIT == 0) return dpp<kQuadXor1>(x);
    else if constexpr (BIT == 1) return dpp<kQuadXor2>(x);
    else if constexpr (BIT == 2) return dpp<kRowHalfMirror>(x);
    else if constexpr (BIT == 3) return dpp<kRowMirror>(x);
    else if constexpr (BIT == 4) return swap16(x);
    else return swap32(x, lane);
}

struct OpSum { __device__ float operator()(float a, float b) const { return a + b; } };
struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// Combine x over all lanes that agree on lane-index bits below LO.
template <int LO, typename Op>
__device__ __forceinline__ float allreduce_from(float x, int lane, Op op) {
    if constexpr (LO <= 0) x = op(x, dpp<kQuadXor1>(x));
    if constexpr (LO <= 1) x = op(x, dpp<kQuadXor2>(x));
    if constexpr (LO <= 2) x = op(x, dpp<kRowRor4>(x));
    if constexpr (LO <= 3) x = op(x, dpp<kRowRor8>(x));
    if constexpr (LO <= 4) x = op(x, swap16(x));
    if constexpr (LO <= 5) x = op(x, swap32(x, lane));
    return x;
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Values the compiler cannot prove wave-uniform are pinned to scalar
// registers; a buffer descriptor built from a per-lane value would be
// wrapped in a waterfall loop around every load.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
    const uint64_t u = (uint64_t)x;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ------------------------------------------------------------------ element types
template <typename DT>
__device__ __forceinline__ float dot_chunk(const u32x4 &q, const u32x4 &k) {
    float acc = 0.f;
    if constexpr (std::is_same_v<DT, BF16>) {
        static_for<0, 4>([&]<int i>() {
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(q[i]), as_bf2(k[i]), acc, false);
        });
    } else if constexpr (std::is_same_v<DT, F16>) {
        static_for<0, 4>([&]<int i>() {
            acc = __builtin_amdgcn_fdot2(as_h2(q[i]), as_h2(k[i]), acc, false);
        });
    } else {
        static_for<0, 4>([&]<int i>() { acc = __builtin_fmaf(as_f(q[i]), as_f(k[i]), acc); });
    }
    return acc;
}

template <typename DT>
__device__ __forceinline__ void chunk_to_f32(const u32x4 &v, float (&f)[16 / DT::kBytes]) {
    if constexpr (std::is_same_v<DT, BF16>) {
        static_for<0, 4>([&]<int i>() {
            f[2 * i] = as_f(v[i] << 16);
            f[2 * i + 1] = as_f(v[i] & 0xFFFF0000u);
        });
    } else if constexpr (std::is_same_v<DT, F16>) {
        static_for<0, 4>([&]<int i>() {
            const f16x2 h = as_h2(v[i]);
            f[2 * i] = (float)h[0];
            f[2 * i + 1] = (float)h[1];
        });
    } else {
        static_for<0, 4>([&]<int i>() { f[i] = as_f(v[i]); });
    }
}

// Round-to-nearest-even store of one output element.
template <typename DT>
__device__ __forceinline__ void store_elem(void *out, int64_t idx, float x) {
    if constexpr (std::is_same_v<DT, BF16>) {
        uint32_t u = as_u(x);
        uint16_t b;
        if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
            b = (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
        } else {
            u += 0x7FFFu + ((u >> 16) & 1u);
            b = (uint16_t)(u >> 16);
        }
        static_cast<uint16_t *>(out)[idx] = b;
    } else if constexpr (std::is_same_v<DT, F16>) {
        static_cast<_Float16 *>(out)[idx] = (_Float16)x;
    } else {
        static_cast<float *>(out)[idx] = x;
    }
}

__device__ __forceinline__ u32x4 load_chunk(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// ------------------------------------------------------------------ partition kernel
template <typename DT, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void attn_partition_kernel(DecodeArgs a) {
    constexpr int EB = DT::kBytes;
    constexpr int VEC = 16 / EB;          // elements per 16-byte chunk
    constexpr int R = D / VEC;            // lanes covering one token row
    constexpr int LOG_R = ilog2(R);
    constexpr int RPL = kWave / R;        // rows per wave load
    constexpr int NI = kSubTile / RPL;    // loads per lane per sub-tile (K and V each)
    constexpr int NP = NI * G;            // q.k partials per lane
    constexpr int LOG_NP = ilog2(NP);
    constexpr int RS = LOG_R < LOG_NP ? LOG_R : LOG_NP;  // reduce-scatter steps
    constexpr int NPL = NP >> RS;         // summed scores per lane afterwards
    constexpr int LOG_G = ilog2(G);
    constexpr int SG = kSubTile * G;      // scores per sub-tile
    constexpr int SPL = (SG + kWave - 1) / kWave;
    static_assert(R >= 1 && R <= kWave && (R & (R - 1)) == 0, "row must map to a power-of-two lane count");
    static_assert(NI >= 1 && NI * RPL == kSubTile, "sub-tile must be whole wave loads");
    static_assert((1 << LOG_G) == G, "group must be a power of two");

    __shared__ float s_lds[NW][SG];       // scores, then probabilities, of the current sub-tile
    __shared__ float a_lds[NW][G];        // per-head rescale factor
    __shared__ float m_lds[NW][G];
    __shared__ float l_lds[NW][G];
    __shared__ float acc_lds[NW][G][D];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = blockIdx.x;
    const int kvh = blockIdx.y;
    const int seq = blockIdx.z;
    const int Hq = a.num_q_heads;
    const int P = a.part_tokens;
    int L = ((const_i32_ptr)a.context_lens)[seq];
    L = L < a.max_context_len ? L : a.max_context_len;
    L = L > 0 ? L : 0;
    const int64_t out_row0 = (int64_t)seq * Hq + (int64_t)kvh * G;  // first q head of the group

    if (L == 0) {  // empty context: the output is the empty sum
        if (part == 0)
            for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave)
                store_elem<DT>(a.out, out_row0 * D + idx, 0.f);
        return;
    }
    const int T0 = part * P;
    if (T0 >= L) return;
    const int nparts = (L + P - 1) / P;
    const int T1 = min(L, T0 + P);
    const int nsub = (T1 - T0 + kSubTile - 1) / kSubTile;

    const int g = lane / R;  // row inside one wave load
    const int c = lane % R;  // 16-byte chunk inside the row

    // q chunks of the G query heads that read this KV head
    u32x4 qr[G];
    {
        const char *qb = static_cast<const char *>(a.q) + (out_row0 * D) * EB + c * 16;
        static_for<0, G>([&]<int h>() { qr[h] = *reinterpret_cast<const u32x4 *>(qb + h * D * EB); });
    }

    const const_i32_ptr table = (const_i32_ptr)(a.block_tables + (int64_t)seq * a.max_blocks_per_seq);
    const int BS = a.block_size;
    const int64_t head_elems = (int64_t)BS * D;
    const int64_t block_elems = (int64_t)a.num_kv_heads * head_elems;
    const char *kc = static_cast<const char *>(a.k_cache);
    const char *vc = static_cast<const char *>(a.v_cache);

    float m_run = -__builtin_inff();   // running max of this lane's head (lane % G)
    float l_run = 0.f;                 // this lane's share of the exp-sum
    float acc[G][VEC];
    static_for<0, G>([&]<int h>() { static_for<0, VEC>([&]<int e>() { acc[h][e] = 0.f; }); });

    // Issues the K and V loads of sub-tile `st`.  A sub-tile past the end of
    // the partition gets an empty buffer range: the loads return zeros without
    // touching memory, so the caller can issue them unconditionally (a
    // conditional load would make the wait counters drain the prefetch).
    auto load_tile = [&](int st, u32x4 (&kr)[NI], u32x4 (&vr)[NI]) {
        const int t0 = T0 + st * kSubTile;
        // rows left in the partition from t0; only the first 16 are ever
        // addressed, so the descriptor needs no upper clamp (a two-sided clamp
        // becomes a VALU med3 whose register hazard drains the load queue)
        int rows = T1 - t0;
        rows = rows > 0 ? rows : 0;
        const int tc = rows > 0 ? t0 : T0;  // keeps the table read inside the row
        const int j = tc / BS;
        const int row0 = tc - j * BS;
        const int64_t phys = table[j];
        const int64_t off = uniform((phys * block_elems + (int64_t)kvh * head_elems + (int64_t)row0 * D) * EB);
        const int nbytes = uniform(rows * D * EB);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(kc + off), 0, nbytes, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)(vc + off), 0, nbytes, kBufferFlags);
        static_for<0, NI>([&]<int i>() { kr[i] = load_chunk(rk, ((i * RPL + g) * D) * EB + c * 16); });
        static_for<0, NI>([&]<int i>() { vr[i] = load_chunk(rv, ((i * RPL + g) * D) * EB + c * 16); });
    };

    auto process_tile = [&](int st, const u32x4 (&kr)[NI], const u32x4 (&vr)[NI]) {
        const int t0 = T0 + st * kSubTile;
        const int nvalid = min(kSubTile, L - t0);
        // ---- q.k partial sums over this lane's chunk, then reduce-scatter across the row
        float pd[NP];
        static_for<0, NI>([&]<int i>() {
            static_for<0, G>([&]<int h>() { pd[i * G + h] = dot_chunk<DT>(qr[h], kr[i]); });
        });
        static_for<0, LOG_R>([&]<int s>() {
            constexpr int bit = LOG_R - 1 - s;
            if constexpr (s < RS) {
                constexpr int half = (NP >> s) / 2;
                const bool hi = (c >> bit) & 1;
                static_for<0, half>([&]<int k>() {
                    const float lo_v = pd[k], hi_v = pd[k + half];
                    const float send = hi ? lo_v : hi_v;
                    const float keep = hi ? hi_v : lo_v;
                    pd[k] = keep + partner<bit>(send, lane);
                });
            } else {
                pd[0] = pd[0] + partner<bit>(pd[0], lane);
            }
        });
        {
            const int jbase = (c >> (LOG_R - RS)) * NPL;
            const bool writer = (c & ((1 << (LOG_R - RS)) - 1)) == 0;
            if (writer) {
                static_for<0, NPL>([&]<int k>() {
                    const int jj = jbase + k;
                    const int tok = (jj / G) * RPL + g;
                    s_lds[wave][tok * G + (jj % G)] = pd[k];
                });
            }
        }
        wave_sync();
        // ---- softmax update in the one-score-per-lane layout (head = lane % G)
        float sv[SPL];
        float tmax = -__builtin_inff();
        static_for<0, SPL>([&]<int u>() {
            const int idx = lane + u * kWave;
            const int tok = idx / G;
            float x = -__builtin_inff();
            if (idx < SG && tok < nvalid) x = s_lds[wave][idx] * a.scale_log2;
            sv[u] = x;
            tmax = fmaxf(tmax, x);
        });
        tmax = allreduce_from<LOG_G>(tmax, lane, OpMax{});
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = fast_exp2(m_run - m_new);
        const bool grew = m_new > m_run;
        m_run = m_new;
        float psum = 0.f;
        static_for<0, SPL>([&]<int u>() {
            const int idx = lane + u * kWave;
            const float p = fast_exp2(sv[u] - m_new);
            psum += p;
            if (idx < SG) s_lds[wave][idx] = p;
        });
        l_run = l_run * alpha + psum;
        if (__builtin_amdgcn_ballot_w64(grew) != 0) {
            if (lane < G) a_lds[wave][lane] = alpha;
            wave_sync();
            static_for<0, G>([&]<int h>() {
                const float al = a_lds[wave][h];
                static_for<0, VEC>([&]<int e>() { acc[h][e] *= al; });
            });
        }
        wave_sync();
        // ---- acc += p * V for the lane's chunk of each of its rows
        static_for<0, NI>([&]<int i>() {
            const int tok = i * RPL + g;
            float pv[G];
            static_for<0, G>([&]<int h>() { pv[h] = s_lds[wave][tok * G + h]; });
            float vf[VEC];
            chunk_to_f32<DT>(vr[i], vf);
            static_for<0, G>([&]<int h>() {
                static_for<0, VEC>([&]<int e>() { acc[h][e] = __builtin_fmaf(pv[h], vf[e], acc[h][e]); });
            });
        });
        wave_sync();
    };

    // ---- main loop: sub-tiles wave, wave+NW, ...; the next tile's loads are
    // always in flight while the current one is consumed
    {
        u32x4 ka[NI], va[NI], kb[NI], vb[NI];
        int st = wave;
        load_tile(st, ka, va);
        while (true) {
            load_tile(st + NW, kb, vb);
            if (st >= nsub) break;
            process_tile(st, ka, va);
            st += NW;
            load_tile(st + NW, ka, va);
            if (st >= nsub) break;
            process_tile(st, kb, vb);
            st += NW;
        }
    }

    // ---- wave totals: exp-sum per head, acc summed over the rows of a load
    const float l_tot = allreduce_from<LOG_G>(l_run, lane, OpSum{});
    static_for<0, G>([&]<int h>() {
        static_for<0, VEC>([&]<int e>() { acc[h][e] = allreduce_from<LOG_R>(acc[h][e], lane, OpSum{}); });
    });
    if (lane < G) {
        m_lds[wave][lane] = m_run;
        l_lds[wave][lane] = l_tot;
    }
    if (g == 0) {
        static_for<0, G>([&]<int h>() {
            static_for<0, VEC>([&]<int e>() { acc_lds[wave][h][c * VEC + e] = acc[h][e]; });
        });
    }
    __syncthreads();

    // ---- merge the waves of this workgroup; finish or hand the partial on
    for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = -__builtin_inff();
        static_for<0, NW>([&]<int w>() { M = fmaxf(M, m_lds[w][h]); });
        float num = 0.f, den = 0.f;
        static_for<0, NW>([&]<int w>() {
            const float sc = fast_exp2(m_lds[w][h] - M);
            num = __builtin_fmaf(sc, acc_lds[w][h][d], num);
            den = __builtin_fmaf(sc, l_lds[w][h], den);
        });
        const int64_t row = out_row0 + h;
        if (nparts == 1) {
            store_elem<DT>(a.out, row * D + d, num / den);
        } else {
            const int64_t pr = row * a.max_parts + part;
            a.ws_acc[pr * D + d] = num;
            if (d == 0) {
                a.ws_ml[pr * 2] = M;
                a.ws_ml[pr * 2 + 1] = den;
            }
        }
    }
}

// ------------------------------------------------------------------ merge kernel
// Per (sequence, q head): out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
constexpr int kReduceThreads = 256;

__device__ float block_reduce(float x, float *scratch, bool is_max) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    x = is_max ? allreduce_from<0>(x, lane, OpMax{}) : allreduce_from<0>(x, lane, OpSum{});
    if (lane == 0) scratch[wave] = x;
    __syncthreads();
    float r = scratch[0];
    for (int w = 1; w < kReduceThreads / 64; ++w) r = is_max ? fmaxf(r, scratch[w]) : r + scratch[w];
    __syncthreads();
    return r;
}

template <typename DT, int D>
__global__ __launch_bounds__(kReduceThreads) void attn_merge_kernel(DecodeArgs a) {
    constexpr int NS = kReduceThreads / D;  // partition slices summed in parallel
    __shared__ float w_lds[kMaxParts];
    __shared__ float part_lds[kReduceThreads];
    __shared__ float scratch[kReduceThreads / 64];
    const int h = blockIdx.x;
    const int seq = blockIdx.y;
    const int P = a.part_tokens;
    int L = a.context_lens[seq];
    L = L < a.max_context_len ? L : a.max_context_len;
    L = L > 0 ? L : 0;
    const int n = (L + P - 1) / P;
    if (n <= 1) return;  // written directly by the partition kernel
    const int64_t row = (int64_t)seq * a.num_q_heads + h;
    const float *ml = a.ws_ml + row * a.max_parts * 2;
    const float *acc = a.ws_acc + row * a.max_parts * D;
    const int tid = threadIdx.x;

    float M = -__builtin_inff();
    for (int p = tid; p < n; p += kReduceThreads) M = fmaxf(M, ml[2 * p]);
    M = block_reduce(M, scratch, true);
    float den = 0.f;
    for (int p = tid; p < n; p += kReduceThreads) {
        const float w = fast_exp2(ml[2 * p] - M);
        w_lds[p] = w;
        den = __builtin_fmaf(w, ml[2 * p + 1], den);
    }
    den = block_reduce(den, scratch, false);  // its barriers also publish w_lds

    const int d = tid % D;
    const int slice = tid / D;
    float num = 0.f;
    for (int p = slice; p < n; p += NS) num = __builtin_fmaf(w_lds[p], acc[(int64_t)p * D + d], num);
    part_lds[tid] = num;
    __syncthreads();
    if (slice == 0) {
        float s = part_lds[d];
        for (int k = 1; k < NS; ++k) s += part_lds[k * D + d];
        store_elem<DT>(a.out, row * D + d, s / den);
    }
}

// ------------------------------------------------------------------ dispatch
constexpr int kWavesPerGroup = 4;

template <typename DT, int D, int G>
hipError_t launch_typed(const DecodeArgs &a, const DecodePlan &plan, hipStream_t stream) {
    const dim3 grid((unsigned)plan.max_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
    attn_partition_kernel<DT, D, G, kWavesPerGroup><<<grid, dim3(kWavesPerGroup * kWave), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.max_parts <= 1) return e;
    attn_merge_kernel<DT, D><<<dim3((unsigned)a.num_q_heads, (unsigned)a.num_seqs), dim3(kReduceThreads), 0, stream>>>(a);
    return hipGetLastError();
}

template <typename DT, int D>
hipError_t launch_group(int group, const DecodeArgs &a, const DecodePlan &plan, hipStream_t s) {
    switch (group) {
        case 1: return launch_typed<DT, D, 1>(a, plan, s);
        case 2: return launch_typed<DT, D, 2>(a, plan, s);
        case 4: return launch_typed<DT, D, 4>(a, plan, s);
        case 8: return launch_typed<DT, D, 8>(a, plan, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename DT>
hipError_t launch_dim(int head_dim, int group, const DecodeArgs &a, const DecodePlan &plan, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_group<DT, 64>(group, a, plan, s);
        case 128: return launch_group<DT, 128>(group, a, plan, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_supported(int32_t dtype, int32_t head_dim, int32_t group) {
    const bool dt = dtype == 0 || dtype == 1 || dtype == 2;
    const bool hd = head_dim == 64 || head_dim == 128;
    const bool gr = group == 1 || group == 2 || group == 4 || group == 8;
    return dt && hd && gr;
}

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                       int32_t max_context_len) {
    DecodePlan p{};
    p.waves = kWavesPerGroup;
    // 256 tokens per workgroup (4 waves x 4 sub-tiles) by default; long
    // contexts take larger partitions so that a sequence has <= 1024 of them.
    int part = 256;
    const int64_t need = ((int64_t)max_context_len + 1023) / 1024;
    while (part < need) part *= 2;
    p.part_tokens = part;
    const int64_t parts = ((int64_t)max_context_len + part - 1) / part;
    p.max_parts = (int32_t)(parts > 1 ? parts : 1);
    if (p.max_parts > 1) {
        const size_t rows = (size_t)num_seqs * (size_t)num_q_heads * (size_t)p.max_parts;
        p.ws_acc_offset = 0;
        const size_t acc_bytes = rows * (size_t)head_dim * sizeof(float);
        p.ws_ml_offset = (acc_bytes + 255) & ~(size_t)255;
        p.workspace_bytes = p.ws_ml_offset + rows * 2 * sizeof(float);
    }
    return p;
}

hipError_t launch_attn_decode(int32_t dtype, int32_t head_dim, int32_t group,
                              const DecodeArgs &a, const DecodePlan &plan, hipStream_t stream) {
    switch (dtype) {
        case 0: return launch_dim<F32>(head_dim, group, a, plan, stream);
        case 1: return launch_dim<F16>(head_dim, group, a, plan, stream);
        case 2: return launch_dim<BF16>(head_dim, group, a, plan, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
