// Split-K differential attention decode for gfx950 (bf16 caches, fp32 math, d = 64, 2d = 128).
//
// Operation (Ultralytics glossary "Differential Transformer", section on how differential attention works): each
// new query token of a (batch, head) attends to the cache with the two softmax maps; output
// sum_j (a_j - lambda b_j) v_j, then optionally the per-head RMS normalisation and the (1 - lambda_init) scale.
//
// The pass is HBM-bound (each cached byte is read once, 1.5 FLOP per byte), so the design is about streaming:
//   * decode_multi_mfma: one wave per (head, key split) holds the T <= 16 new tokens of the head (T = 1 for plain
//     decode) in the 16 columns of 16x16x32 MFMA tiles: scores K Q^T and outputs V^T P^T on the matrix cores, an
//     online softmax per query in between (see the kernel).  New token t sits at cache position len - T + t and
//     sees the keys up to its own position.  The split's state (m, l, O[128]) per map and query goes to the
//     workspace.
//   * decode_merge: one wave per (head, query) merges the splits by log-sum-exp and applies the epilogue; with
//     many splits, decode_merge_groups first merges groups of them.
//   * Ragged caches: with a per-sequence length array, sequence b uses the first lens[b] cache rows (the cache is
//     padded to L rows).  With enough (sequence, head) items the keys of all of them are cut into equal ranges, one
//     per wave, whatever the lengths (decode_ragged_mfma, decode_ragged_merge); otherwise the fixed split plan runs,
//     and its splits past a sequence's end write an empty state (max -inf, sum 0), which the merge weighs by 0.
//   * Paged caches (template flag PAGED): a sequence's rows live in fixed-size pages of a pool shared by all
//     sequences, found through a per-sequence block table.  A split first copies its page indices into LDS
//     (stage_pages); every row address then goes through cache_elem.
//   * Padded caches are addressed through per-tensor batch, head and row strides (dense ones included), so K1, K2
//     and V may be views of token-major or packed buffers.
#include <algorithm>

#include "launch.h"

namespace diffattn {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int D = 64;
constexpr int DV = 128;
constexpr int MAX_SPLIT_KEYS = 8192;   // keys per split (the kernel keeps no per-key state)
constexpr int PT_MAX = 520;            // page-table entries staged per split
static_assert(MAX_SPLIT_KEYS / 16 + 2 <= PT_MAX, "a split spans at most keys / 16 + 2 pages");
constexpr int PART_FLOATS = 4 + 2 * DV;       // m1, l1, m2, l2, O1[128], O2[128]
static_assert(PART_FLOATS == PARTIAL_FLOATS, "the decode's split states are the shared partial-state format");
constexpr int MAX_T = 16;                     // new tokens per sequence in multi-token decode
constexpr float LOG2E = 1.4426950408889634f;

struct SplitPlan {
    int splits;      // key splits per head
    int split_keys;  // keys per split (the last split may be shorter)
};

__host__ __device__ inline SplitPlan plan_splits(int64_t BH, int64_t L, int64_t max_keys, int64_t min_grid) {
    // At least ceil(L / max_keys) splits; more for few heads so that the grid has >= ~min_grid workgroups,
    // but never below 64 keys per split.
    int64_t s = (L + max_keys - 1) / max_keys;
    const int64_t want = (min_grid + BH - 1) / (BH > 0 ? BH : 1);
    const int64_t cap = (L + 63) / 64;
    if (s < want) s = want < cap ? want : cap;
    if (s < 1) s = 1;
    int64_t keys = (L + s - 1) / s;
    s = (L + keys - 1) / keys;  // no empty split
    return SplitPlan{(int)s, (int)keys};
}

// Paged caches: copy the block-table entries of ENTRIES pages of sequence b, from the one holding row j0 on,
// into ptab (clamped to the pool; positions past the table repeat its last entry), so that a row's page is an LDS
// read rather than a dependent global load.  Returns the first staged page.  The caller makes the writes visible
// (a barrier, or the same wave's later reads).
template <bool PAGED, int ENTRIES>
__device__ __forceinline__ int stage_pages(const DecodePages& pg, int b, int j0, int* ptab, int tid, int nthreads) {
    if constexpr (!PAGED) {
        return 0;
    } else {
        const int pg0 = j0 >> pg.log2_page;
        for (int i = tid; i < ENTRIES; i += nthreads) {
            const int idx = min(pg0 + i, pg.max_pages - 1);
            ptab[i] = min(max(pg.table[(size_t)b * pg.max_pages + idx], 0), pg.num_pages - 1);
        }
        return pg0;
    }
}
// Element offset of cache row r (logical position in its sequence) of head hh of sequence b in cache tensor t (width
// elements per row): padded caches through their strides, paged pools [num_pages][H][page][width] through the
// staged page indices.
template <bool PAGED>
__device__ __forceinline__ int64_t cache_elem(const DecodePages& pg, const CacheStrides& cs, const int* ptab, int pg0,
                                              int b, int hh, int H, int r, int t, int width) {
    if constexpr (!PAGED) {
        return b * cs.b[t] + hh * cs.h[t] + (int64_t)r * cs.n[t];
    } else {
        const int page = ptab[(r >> pg.log2_page) - pg0];
        return (int64_t)((((size_t)page * H + hh) << pg.log2_page) + (r & ((1 << pg.log2_page) - 1))) * width;
    }
}

// Cache length of sequence b: lens[b] clamped to [lo, L], or L without a length array.
__device__ __forceinline__ int seq_len(const int* lens, int b, int lo, int L) {
    return lens ? min(max(lens[b], lo), L) : L;
}

// 16-byte nontemporal load (cache policy "nt": streamed data that will not be read again).
__device__ __forceinline__ u32x4 ldnt(const uint16_t* p) { return __builtin_nontemporal_load((const u32x4*)p); }

// One wave per (head, query): blockIdx.x = bh * T + t.  Every query sees at least one key, so some split is
// non-empty and the merged maxima are finite.
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ ws, uint16_t* __restrict__ gout,
                                                          int splits, int T, Epilogue ep) {
    const int item = blockIdx.x;
    merge_partial_row(ws + (size_t)item * splits * PART_FLOATS, splits, ep, item / T, gout + (size_t)item * DV,
                      (int)threadIdx.x);
}

// First level of the merge for many splits: wave (item, g) merges splits [g group, (g + 1) group) of its item
// (item = bh * T + t) into one state at ws2[item][g]; decode_merge_kernel then merges the groups' states.
__global__ __launch_bounds__(64) void decode_merge_groups_kernel(const float* __restrict__ ws, float* __restrict__ ws2,
                                                                 int splits, int group, int groups) {
    const int64_t item = blockIdx.x / groups;
    const int g = (int)(blockIdx.x % groups);
    const int s0 = g * group;
    merge_partial_state(ws + (item * splits + s0) * PART_FLOATS, min(group, splits - s0),
                        ws2 + (item * groups + g) * PART_FLOATS, (int)threadIdx.x);
}

// Splits per item merged by one wave in one pass; beyond that, two levels of about sqrt(splits) states each.
constexpr int MERGE_DIRECT_MAX = 32;
struct MergePlan {
    int group, groups;   // splits per first-level group, groups per item (1: a single merge pass)
};
MergePlan merge_plan(int splits) {
    if (splits <= MERGE_DIRECT_MAX) return MergePlan{splits, 1};
    int g = 1;
    while (g * g < splits) ++g;
    return MergePlan{g, (splits + g - 1) / g};
}

template <bool V> struct Flag { static constexpr bool value = V; };

// Multi-token split on the matrix cores: one wave per (head, key split), all T <= 16 queries of the head as the 16
// columns of v_mfma_f32_16x16x32_bf16 tiles (A 16 x 32: lane holds A[m = l % 16][k = 8 (l / 16) + j]; B 32 x 16:
// lane holds B[k = 8 (l / 16) + j][n = l % 16]; D 16 x 16: lane holds D[m = 4 (l / 16) + i][n = l % 16]).
//   * Scores S^T = K Q^T per 32-key tile: A = K rows, loaded from global memory straight into the operand layout
//     (each lane 16 bytes of one key row per operand), B = the queries.  Lane l then holds query t = l % 16 and keys
//     4 g + i, 16 + 4 g + i of the tile (g = l / 16), which are, in order, its 8 probabilities as the B operand of
//     O^T = V^T P^T.
//   * V rows are loaded into registers (16 lanes per 256-byte row, nontemporal) and written to the wave's one 8 KiB
//     LDS tile; each V^T A operand (one channel, the lane's 8 keys) is two ds_read_b64_tr_b16 reads of it.  The next
//     tile's rows are loaded while this one is computed.  With no K in LDS a wave needs 8 KiB of it, so the register
//     file, not the LDS, sets the occupancy (two waves per SIMD).
//   * Splits are long (up to 8192 keys, see plan_call): fewer, longer streams read faster here.
//   * Online softmax per query and map, offsets moved only when a tile's max exceeds them by more than 2^8 (so no
//     probability exceeds 2^8); offsets start at -FLT_MAX so a query with no visible key in the split keeps an empty
//     state without NaN.  The split's state per query goes to the workspace in the merge kernel's format.
constexpr int MT = 32;                 // keys per tile
constexpr int MV_TILE = MT * DV * 2;   // 8 KiB
constexpr float MULTI_RESCALE = 8.0f;  // log2 units

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)a) |
           ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)b) << 16);
}
// Combine a per-lane value over the four lanes holding one query column (l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float col_max(float x) {
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float col_sum(float x) {
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
// Raw V tile in LDS: row r (key) of 256 bytes, chunk c at c ^ mv_sw(r).  A transposing (64-bit) read is served in
// windows of 32 consecutive lanes, here 8 rows x 2 adjacent chunks; mv_sw, linear over GF(2) in the bits of r % 16
// (found by exhaustive search over such maps), puts those 16 chunks on 16 distinct bank quads.
__device__ __forceinline__ int mv_sw(int r) {
    return ((r & 1) << 3) ^ (((r >> 1) & 1) << 2) ^ (((r >> 2) & 1) * 3) ^ (((r >> 3) & 1) << 1);
}
__device__ __forceinline__ int mv_off(int row, int chunk) { return row * 256 + ((chunk ^ mv_sw(row)) << 4); }
struct MultiMap {
    float m, l;   // running offset (log2 units of the scaled scores) and this lane's part of the sum
};

// One map's tile: scores (already scaled to log2 units, masked -inf) -> packed probabilities; moves the offset
// (and rescales O and l) when the tile's column max exceeds it by more than MULTI_RESCALE.
__device__ __forceinline__ bf16x8 multi_softmax(const f32x4 (&s)[2], MultiMap& st, f32x4 (&o)[8]) {
    const float x = col_max(fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                                  fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3]))));
    if (__any(x > st.m + MULTI_RESCALE)) {
        const float mn = fmaxf(st.m, x);
        const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
        st.m = mn;
        st.l *= alpha;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[cb][i] *= alpha;
    }
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(s[e >> 2][e & 3] - st.m);
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack_bf16(p[2 * k], p[2 * k + 1]);
    // The sum is taken in fp32 with plain VALU adds: v_dot2 on the packed values would run on the matrix pipe,
    // behind the value MFMAs.
    st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    return __builtin_bit_cast(bf16x8, w);
}

// The states of one split: keys [j0, j0 + n) (n >= 1) of head bh (sequence bb, head hh; Lb cache rows, the T new
// tokens at positions Lb - T ..) against the T queries.  Query t's state goes to dst0[(t stride + sp) PART_FLOATS ..].
// vs and ptab are the calling wave's LDS (the V tile and the staged page indices).
template <bool PAGED>
__device__ __forceinline__ void split_states(const uint16_t* __restrict__ gq1, const uint16_t* __restrict__ gk1,
                                             const uint16_t* __restrict__ gq2, const uint16_t* __restrict__ gk2,
                                             const uint16_t* __restrict__ gv, float* __restrict__ dst0, int stride,
                                             int sp, int bh, int bb, int hh, int H, int Lb, int j0, int n, int T,
                                             const DecodePages& pg, const CacheStrides& cs, unsigned char* vs,
                                             int* ptab) {
    const int lane = threadIdx.x;
    const int g = lane >> 4, l16 = lane & 15;
    const int pos0 = Lb - T;                                 // cache position of query 0
    const float c = LOG2E * 0.125f;
    const int t_col = l16;                                   // this lane's query column
    const bool t_ok = t_col < T;

    // Queries as B operands (k = feature 32 kh + 8 g + j, n = query); columns t >= T are zero.
    bf16x8 qa[2], qb[2];
    {
        const int tq = min(t_col, T - 1);   // every lane loads (no divergent branch); columns t >= T are zeroed
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            u32x4 a = *(const u32x4*)(gq1 + ((size_t)bh * T + tq) * D + 32 * kh + 8 * g);
            u32x4 b = *(const u32x4*)(gq2 + ((size_t)bh * T + tq) * D + 32 * kh + 8 * g);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                a[k] = t_ok ? a[k] : 0u;
                b[k] = t_ok ? b[k] : 0u;
            }
            qa[kh] = __builtin_bit_cast(bf16x8, a);
            qb[kh] = __builtin_bit_cast(bf16x8, b);
        }
    }

    // Cache row index of absolute row r of this sequence.  Paged caches read the page index from the split's staged
    // table (LDS), so no global load stands in front of a tile's loads.  One wave: its own later reads see the table.
    const int pg0 = stage_pages<PAGED, PT_MAX>(pg, bb, j0, ptab, lane, 64);
    auto elem = [&](int r, int t, int width) __attribute__((always_inline)) -> int64_t {
        return cache_elem<PAGED>(pg, cs, ptab, pg0, bb, hh, H, r, t, width);
    };

    // Tile loads (rows past the split's end repeat its last row and are masked), into registers.
    //   K1 and K2 go straight into the layout of the A operand of S^T = K Q^T: for key block kb and feature half kh,
    //   lane l holds key row 16 kb + l16 of the tile, features 32 kh + 8 g .. + 7.
    //   V rows are staged through LDS for the transposing reads: lane L holds key 4 p + L / 16, 16-byte chunk L % 16
    //   (p = 0..7), written to LDS at mv_off(row, chunk).
    const int n_tiles = (n + MT - 1) / MT;
    u32x4 ka[2][2], kb2[2][2], vw[8];
    auto load_k = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int r = min(tile * MT + 16 * kb + l16, n - 1);
            const int64_t e1 = elem(j0 + r, C_K1, D), e2 = elem(j0 + r, C_K2, D);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                ka[kb][kh] = *(const u32x4*)(gk1 + e1 + 32 * kh + 8 * g);
                kb2[kb][kh] = *(const u32x4*)(gk2 + e2 + 32 * kh + 8 * g);
            }
        }
    };
    auto load_v = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int r = min(tile * MT + 4 * p + (lane >> 4), n - 1);
            vw[p] = ldnt(gv + elem(j0 + r, C_V, DV) + 8 * (lane & 15));
        }
    };
    auto store_v = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 8; ++p) *(u32x4*)(vs + mv_off(4 * p + (lane >> 4), lane & 15)) = vw[p];
    };

    // V^T operand offsets: lane 4 jj + qq of 16-lane group g supplies row 4 g + jj (then 16 + 4 g + jj), channels
    // 16 cb + 4 qq .. + 3, and receives channel 16 cb + l16 of those 4 keys; cb XORs 32 cb into the offset.
    const int jj = (lane >> 2) & 3, qq = lane & 3;
    const int v_rd0 = mv_off(4 * g + jj, qq >> 1) + 8 * (qq & 1);
    auto v_frag = [&](const unsigned char* slot, int cb) __attribute__((always_inline)) {
        const unsigned char* p = slot + (v_rd0 ^ (32 * cb));
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * 256));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x4 o1[8], o2[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) { o1[cb][i] = 0.f; o2[cb][i] = 0.f; }
    MultiMap st1 = {-__FLT_MAX__, 0.f}, st2 = st1;

    load_v(0);
    load_k(0);
    // Q must have landed before the loop: the compiler waits for it here (and with it for tile 0's loads, issued
    // after it), so it places no wait for Q inside the loop.
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) asm volatile("" ::"v"(qa[kh]), "v"(qb[kh]));
    // One tile per step.  The next tile's V rows are loaded as soon as this tile's are in LDS, and its K rows as soon
    // as this tile's scores are issued, so a tile's loads have one whole step to land.  PREFETCH is compile-time (the
    // last tile is peeled), so the loop has no branch around the loads and the compiler's waits stay exact.  This
    // wave alone uses its LDS tile, and its LDS operations complete in order, so no barrier or extra wait orders the
    // next step's writes after this step's reads.
    auto step = [&](auto PREFETCH, int tile) __attribute__((always_inline)) {
        constexpr bool pf = decltype(PREFETCH)::value;
        store_v();
        if constexpr (pf) load_v(tile + 1);
        f32x4 s1[2], s2[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) { s1[kb][i] = 0.f; s2[kb][i] = 0.f; }
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                s1[kb] = mfma16(__builtin_bit_cast(bf16x8, ka[kb][kh]), qa[kh], s1[kb]);
                s2[kb] = mfma16(__builtin_bit_cast(bf16x8, kb2[kb][kh]), qb[kh], s2[kb]);
            }
        }
        if constexpr (pf) load_k(tile + 1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = tile * MT + 16 * kb + 4 * g + i;
                const bool vis = t_ok && r < n && j0 + r <= pos0 + t_col;
                s1[kb][i] = vis ? s1[kb][i] * c : -INFINITY;
                s2[kb][i] = vis ? s2[kb][i] * c : -INFINITY;
            }
        const bf16x8 p1 = multi_softmax(s1, st1, o1);
        const bf16x8 p2 = multi_softmax(s2, st2, o2);
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            const bf16x8 va = v_frag(vs, cb);
            o1[cb] = mfma16(va, p1, o1[cb]);
            o2[cb] = mfma16(va, p2, o2[cb]);
        }
    };
    int tile = 0;
    for (; tile + 1 < n_tiles; ++tile) step(Flag<true>{}, tile);
    step(Flag<false>{}, tile);

    // The split's state per query column: offsets, sums over the column's four lanes, and O (lane holds channels
    // 16 cb + 4 g + i of its column).
    const float l1 = col_sum(st1.l), l2 = col_sum(st2.l);
    if (t_ok) {
        float* dst = dst0 + ((size_t)t_col * stride + sp) * PART_FLOATS;
        if (g == 0) {
            dst[0] = l1 > 0.f ? st1.m : -INFINITY;
            dst[1] = l1;
            dst[2] = l2 > 0.f ? st2.m : -INFINITY;
            dst[3] = l2;
        }
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            *(f32x4*)(dst + 4 + 16 * cb + 4 * g) = o1[cb];
            *(f32x4*)(dst + 4 + DV + 16 * cb + 4 * g) = o2[cb];
        }
    }
}

// Fixed split plan: one wave per (head, key split) = (blockIdx.x / splits, blockIdx.x % splits); splits past their
// sequence's end write an empty state (max -inf, sum 0), which the merge weighs by 0.
template <bool PAGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_multi_mfma_kernel(
    const uint16_t* __restrict__ gq1, const uint16_t* __restrict__ gk1, const uint16_t* __restrict__ gq2,
    const uint16_t* __restrict__ gk2, const uint16_t* __restrict__ gv, float* __restrict__ ws, int L, int T,
    int splits, int split_keys, const int* __restrict__ lens, int H, DecodePages pg, CacheStrides cs) {
    __shared__ __attribute__((aligned(16))) unsigned char vs[MV_TILE];   // the V tile being used
    __shared__ int ptab[PAGED ? PT_MAX : 1];   // paged caches: the split's page indices
    const int lane = threadIdx.x;
    const int bh = blockIdx.x / splits;
    const int sp = blockIdx.x % splits;
    const int Lb = seq_len(lens, bh / H, T, L);
    const int j0 = sp * split_keys;
    const int n = min(Lb, j0 + split_keys) - j0;
    float* dst0 = ws + (size_t)bh * T * splits * PART_FLOATS;
    if (n <= 0) {
        for (int t = 0; t < T; ++t) {
            float* dst = dst0 + ((size_t)t * splits + sp) * PART_FLOATS;
            if (lane == 0) {
                dst[0] = -INFINITY;
                dst[1] = 0.f;
                dst[2] = -INFINITY;
                dst[3] = 0.f;
            }
            for (int k = lane; k < 2 * DV; k += 64) dst[4 + k] = 0.f;
        }
        return;
    }
    split_states<PAGED>(gq1, gk1, gq2, gk2, gv, dst0, splits, sp, bh, bh / H, bh % H, H, Lb, j0, n, T, pg, cs, vs,
                        ptab);
}

// Balanced plan for ragged caches.  The W = H * sum_b len_b keys of all (sequence, head) items, taken item by item
// (bh = b H + h) and in key order within an item, are cut into ranges of `chunk` keys, one per wave: wave w takes
// keys [w chunk, (w + 1) chunk) of that order, which may end one item and start the next, so every wave streams the
// same number of keys whatever the lengths.  Item bh starts at P = H pre[b] + h len_b (pre: the lengths' exclusive
// prefix sums); waves P / chunk .. (P + len_b - 1) / chunk hold its keys, and wave w writes its state for the item
// to slot w - P / chunk.  chunk >= chunk_min = ceil(L / (RAGGED_SLOTS - 1)) bounds the slots per item by
// (L - 1) / chunk_min + 2 <= RAGGED_SLOTS.  The split and merge kernels derive the same cut from the lengths.
constexpr int RAGGED_MAX_B = 512;     // sequences: one wave scans their lengths (8 per lane)
constexpr int RAGGED_MIN_BH = 128;    // fewer items: the fixed plan's many short splits keep more waves busy
// Waves of the cut: one per SIMD, more if chunks would exceed MAX_SPLIT_KEYS.  Measured at B64 H16 on caches of
// 4K-8K rows: 512, 768 and 1024 waves within 1% of each other (T = 4: 515 us), 1536 3% and 2048 5% slower.
constexpr int RAGGED_WAVES = 1024;
constexpr int RAGGED_SLOTS = MERGE_DIRECT_MAX;
struct RaggedCut {
    int64_t total, chunk;   // keys of all items, keys per wave
};
// By one wave: pre[0..B] (LDS) and the cut.  The caller makes pre visible before reading it (a barrier), and reads
// it through pre_at, so that the values, uniform across the wave, stay scalar (cache addresses derive from them).
__device__ __forceinline__ RaggedCut ragged_cut(const int* __restrict__ lens, int B, int H, int T, int L, int waves,
                                                int chunk_min, int* pre) {
    const int lane = threadIdx.x;
    int carry = 0;   // at most RAGGED_MAX_B * L keys: fits
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int b = b0 + lane;
        int x = b < B ? seq_len(lens, b, T, L) : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (b < B) pre[b + 1] = carry + x;
        carry += __builtin_amdgcn_readlane(x, 63);
    }
    if (lane == 0) pre[0] = 0;
    const int64_t total = (int64_t)H * carry;
    return RaggedCut{total, max((total + waves - 1) / waves, (int64_t)chunk_min)};
}

__device__ __forceinline__ int pre_at(const int* pre, int i) { return __builtin_amdgcn_readfirstlane(pre[i]); }

template <bool PAGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_ragged_mfma_kernel(
    const uint16_t* __restrict__ gq1, const uint16_t* __restrict__ gk1, const uint16_t* __restrict__ gq2,
    const uint16_t* __restrict__ gk2, const uint16_t* __restrict__ gv, float* __restrict__ ws, int L, int T, int B,
    int H, int waves, int chunk_min, int slots, const int* __restrict__ lens, DecodePages pg, CacheStrides cs) {
    __shared__ __attribute__((aligned(16))) unsigned char vs[MV_TILE];
    __shared__ int ptab[PAGED ? PT_MAX : 1];
    __shared__ int pre[RAGGED_MAX_B + 1];
    const RaggedCut cut = ragged_cut(lens, B, H, T, L, waves, chunk_min, pre);
    __syncthreads();
    const int w = blockIdx.x;
    const int64_t start = (int64_t)w * cut.chunk;
    if (start >= cut.total) return;
    const int64_t end = min(start + cut.chunk, cut.total);
    // The item holding key `start`: the last sequence b with H pre[b] <= start, then the head and the offset.
    int b = 0;
    for (int hi = B - 1; b < hi;) {
        const int mid = (b + hi + 1) >> 1;
        if ((int64_t)H * pre_at(pre, mid) <= start) b = mid;
        else hi = mid - 1;
    }
    int64_t item0 = (int64_t)H * pre_at(pre, b);
    int len = pre_at(pre, b + 1) - pre_at(pre, b);
    int h = (int)((start - item0) / len);
    int off = (int)(start - item0 - (int64_t)h * len);
    for (int64_t pos = start;;) {
        const int n = (int)min((int64_t)(len - off), end - pos);
        const int64_t P = item0 + (int64_t)h * len;
        const int bh = b * H + h;
        split_states<PAGED>(gq1, gk1, gq2, gk2, gv, ws + (size_t)bh * T * slots * PART_FLOATS, slots,
                            (int)(w - P / cut.chunk), bh, b, h, H, len, off, n, T, pg, cs, vs, ptab);
        pos += n;
        if (pos >= end) break;
        // More keys in this wave's range: the next item (there is one, since pos < total).
        off = 0;
        if (++h == H) {
            h = 0;
            ++b;
            item0 = (int64_t)H * pre_at(pre, b);
            len = pre_at(pre, b + 1) - pre_at(pre, b);
        }
    }
}

// One wave per (head, query) item = bh * T + t: its slots of the balanced cut merged as decode_merge_kernel does.
__global__ __launch_bounds__(64) void decode_ragged_merge_kernel(const float* __restrict__ ws, uint16_t* __restrict__ gout,
                                                                 int L, int T, int B, int H, int waves, int chunk_min,
                                                                 int slots, const int* __restrict__ lens, Epilogue ep) {
    __shared__ int pre[RAGGED_MAX_B + 1];
    const RaggedCut cut = ragged_cut(lens, B, H, T, L, waves, chunk_min, pre);
    __syncthreads();
    const int item = blockIdx.x;
    const int bh = item / T, b = bh / H, h = bh % H;
    const int len = pre_at(pre, b + 1) - pre_at(pre, b);
    const int64_t P = (int64_t)H * pre_at(pre, b) + (int64_t)h * len;
    const int nseg = (int)((P + len - 1) / cut.chunk - P / cut.chunk + 1);
    merge_partial_row(ws + (size_t)item * slots * PART_FLOATS, nseg, ep, bh, gout + (size_t)item * DV,
                      (int)threadIdx.x);
}

struct RaggedPlan {
    int waves, chunk_min, slots;
};
// The balanced plan's launch, or false where the fixed plan serves (too many sequences to scan, too few items, or
// caches so long that chunk_min would exceed MAX_SPLIT_KEYS).
bool ragged_plan(int64_t BH, int64_t H, int64_t L, RaggedPlan& rp) {
    if (BH <= 0 || H <= 0 || L <= 0) return false;
    if (BH / H > RAGGED_MAX_B || BH < RAGGED_MIN_BH) return false;
    const int64_t chunk_min = (L + RAGGED_SLOTS - 2) / (RAGGED_SLOTS - 1);
    if (chunk_min > MAX_SPLIT_KEYS) return false;
    const int64_t waves = std::max<int64_t>(RAGGED_WAVES, (BH * L + MAX_SPLIT_KEYS - 1) / MAX_SPLIT_KEYS);
    if (waves > 0x7fffffff) return false;
    rp = RaggedPlan{(int)waves, (int)chunk_min, (int)((L - 1) / chunk_min + 2)};
    return true;
}
static_assert(RAGGED_SLOTS <= MERGE_DIRECT_MAX, "one merge pass per item");

// Split plan of a call.  The kernel keeps no per-key state, so splits may be long; fewer, longer splits stream
// faster than many short ones, down to about a wave per SIMD.  Measured at one token on full caches (4 GiB at
// B64 H16 L8192 or B16 H16 L32768, 0.5 GiB at B1 H16 L65536, B1 H1 L1M or B8 H16 L8192): splits of at most 4096
// keys with at least ~512 waves were the fastest or within 1% of it (B64 H16 L8192: 640 us against 652 for one
// 8192-key split per head; B1 H16 L65536: 89 us against 94 for at least 1024 waves).  Several tokens
// take splits of up to 8192 keys and ~1024 waves.  On ragged caches this fixed plan leaves waves of unequal length
// (B64 H16, caches of 4K-8K rows, T = 4: splits of 1024 keys 5.1 TB/s, 2048 5.7, 4096 5.85, one 8192-key split per
// head 5.93); the balanced plan (ragged_plan) serves those calls where it applies: 6.4 TB/s there.
SplitPlan plan_call(int64_t BH, int64_t L, int T) {
    return T == 1 ? plan_splits(BH, L, MAX_SPLIT_KEYS / 2, 512) : plan_splits(BH, L, MAX_SPLIT_KEYS, 1024);
}

}  // namespace

size_t decode_bf16_workspace_bytes(int64_t BH, int64_t H, int64_t L, int T, bool ragged) {
    if (BH <= 0 || L <= 0 || T < 1 || T > MAX_T) return 0;
    const SplitPlan p = plan_call(BH, L, T);
    const MergePlan m = merge_plan(p.splits);
    const size_t states = (size_t)p.splits + (m.groups > 1 ? (size_t)m.groups : 0);
    size_t bytes = (size_t)BH * (size_t)T * states * PART_FLOATS * sizeof(float);
    RaggedPlan rp;
    if (ragged && ragged_plan(BH, H, L, rp))
        bytes = std::max(bytes, (size_t)BH * (size_t)T * (size_t)rp.slots * PART_FLOATS * sizeof(float));
    return bytes;
}

hipError_t launch_decode_bf16_d64(const uint16_t* q1, const uint16_t* k1, const uint16_t* q2, const uint16_t* k2,
                                  const uint16_t* v, uint16_t* out, int64_t BH, int64_t H, int64_t L, int T,
                                  const int* lens, const DecodePages* pages, const CacheStrides& cs, Epilogue ep,
                                  void* workspace, hipStream_t stream) {
    if (T < 1 || T > MAX_T || BH * T > 0x7fffffff) return hipErrorInvalidValue;
    if (pages && ((int64_t)pages->max_pages << pages->log2_page) != L) return hipErrorInvalidValue;
    float* ws = (float*)workspace;
    const DecodePages pg = pages ? *pages : DecodePages{nullptr, 0, 0, 0};
    RaggedPlan rp;
    if (lens && ragged_plan(BH, H, L, rp)) {
        const int B = (int)(BH / H);
        if (pages)
            hipLaunchKernelGGL(decode_ragged_mfma_kernel<true>, dim3((unsigned)rp.waves), dim3(64), 0, stream, q1, k1,
                               q2, k2, v, ws, (int)L, T, B, (int)H, rp.waves, rp.chunk_min, rp.slots, lens, pg, cs);
        else
            hipLaunchKernelGGL(decode_ragged_mfma_kernel<false>, dim3((unsigned)rp.waves), dim3(64), 0, stream, q1, k1,
                               q2, k2, v, ws, (int)L, T, B, (int)H, rp.waves, rp.chunk_min, rp.slots, lens, pg, cs);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(decode_ragged_merge_kernel, dim3((unsigned)(BH * T)), dim3(64), 0, stream,
                           (const float*)ws, out, (int)L, T, B, (int)H, rp.waves, rp.chunk_min, rp.slots, lens, ep);
        return hipGetLastError();
    }
    const SplitPlan p = plan_call(BH, L, T);
    const MergePlan m = merge_plan(p.splits);
    const int64_t blocks = BH * (int64_t)p.splits;
    if (blocks > 0x7fffffff || BH * T * m.groups > 0x7fffffff) return hipErrorInvalidValue;
    if (pages)
        hipLaunchKernelGGL(decode_multi_mfma_kernel<true>, dim3((unsigned)blocks), dim3(64), 0, stream, q1, k1, q2, k2,
                           v, ws, (int)L, T, p.splits, p.split_keys, lens, (int)H, pg, cs);
    else
        hipLaunchKernelGGL(decode_multi_mfma_kernel<false>, dim3((unsigned)blocks), dim3(64), 0, stream, q1, k1, q2,
                           k2, v, ws, (int)L, T, p.splits, p.split_keys, lens, (int)H, pg, cs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (m.groups == 1) {
        hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(BH * T)), dim3(64), 0, stream, (const float*)ws, out,
                           p.splits, T, ep);
    } else {
        // The groups' states follow the splits' states in the workspace.
        float* ws2 = ws + (size_t)BH * T * p.splits * PART_FLOATS;
        hipLaunchKernelGGL(decode_merge_groups_kernel, dim3((unsigned)(BH * T * m.groups)), dim3(64), 0, stream,
                           (const float*)ws, ws2, p.splits, m.group, m.groups);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(BH * T)), dim3(64), 0, stream, (const float*)ws2, out,
                           m.groups, T, ep);
    }
    return hipGetLastError();
}

}  // namespace diffattn
