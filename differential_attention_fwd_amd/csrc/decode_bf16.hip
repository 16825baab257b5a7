// Split-K differential attention decode for gfx950 (bf16 caches, fp32 math, d = 64, 2d = 128).
//
// Operation (Ultralytics glossary "Differential Transformer", section on how differential attention works): one
// query token per (batch, head) attends to the whole cache with the two softmax maps; output
// sum_j (a_j - lambda b_j) v_j, then optionally the per-head RMS normalisation and the (1 - lambda_init) scale.
//
// The pass is HBM-bound (each cached byte is read once, 1.5 FLOP per byte), so the design is about streaming:
//   * decode_split: one workgroup per (head, key split).  Phase 1 reads K1 and K2 rows with 16-byte loads, eight
//     lanes per 128-byte row so every wave-wide load covers 1 KiB of contiguous cache, and keeps the split's
//     scores in LDS.  Phase 2 takes the split's exact maximum and sum per map.  Phase 3 streams V rows (sixteen
//     lanes per 256-byte row) and accumulates both maps' partial outputs in fp32.  The split's state
//     (m, l, O[128]) per map goes to the workspace.
//   * decode_merge: one wave per head merges the splits by log-sum-exp and applies the epilogue.
//   * Ragged caches: with a per-sequence length array, sequence b uses the first lens[b] cache rows (the cache is
//     padded to L rows); splits past its end write an empty state (max -inf, sum 0), which the merge weighs by 0.
//   * decode_multi_split: T > 1 new tokens per sequence (T <= 16), query t at cache position len - T + t seeing
//     keys up to its own position.  The T queries sit in LDS; the split's scores for all of them are kept in LDS
//     (T x keys <= 2048 per map); waves take queries t = wave, wave + 4, ... for the softmax and value passes, so
//     V rows are re-read per query from cache rather than from HBM.
//   * Paged caches (template flag PAGED): a sequence's rows live in fixed-size pages of a pool shared by all
//     sequences, found through a per-sequence block table; every row address goes through cache_row.
#include "launch.h"

namespace diffattn {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int D = 64;
constexpr int DV = 128;
constexpr int THREADS = 256;
constexpr int MAX_SPLIT_KEYS = 1024;          // keys per split (scores of both maps fit in 8 KiB of LDS)
constexpr int PART_FLOATS = 4 + 2 * DV;       // m1, l1, m2, l2, O1[128], O2[128]
constexpr int MAX_T = 16;                     // new tokens per sequence in multi-token decode
constexpr int MULTI_SCORES = 2048;            // T x split keys per map held in LDS by the multi-token kernel
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Note: the vector element is copied to a scalar before __builtin_bit_cast; bit-casting a subscripted vector
// element directly (bit_cast(T, v[k])) compiles to element 0 for every k with this compiler.
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const unsigned ak = a[k], bk = b[k];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ak), __builtin_bit_cast(bf16x2, bk), acc,
                                              false);
    }
    return acc;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s);
    return x;
}

struct SplitPlan {
    int splits;      // key splits per head
    int split_keys;  // keys per split (the last split may be shorter)
};

__host__ __device__ inline SplitPlan plan_splits(int64_t BH, int64_t L) {
    // At least ceil(L / MAX_SPLIT_KEYS) splits; more for few heads so that the grid has >= ~2048 workgroups,
    // but never below 64 keys per split.
    int64_t s = (L + MAX_SPLIT_KEYS - 1) / MAX_SPLIT_KEYS;
    const int64_t want = (2048 + BH - 1) / (BH > 0 ? BH : 1);
    const int64_t cap = (L + 63) / 64;
    if (s < want) s = want < cap ? want : cap;
    if (s < 1) s = 1;
    int64_t keys = (L + s - 1) / s;
    s = (L + keys - 1) / keys;  // no empty split
    return SplitPlan{(int)s, (int)keys};
}

// Index of cache row r (logical position in its sequence) of head bh, in rows of the cache tensors: contiguous
// [B][H][L][w], or paged pools [num_pages][H][page][w] through the block table (entries clamped to the pool).
template <bool PAGED>
__device__ __forceinline__ size_t cache_row(const DecodePages& pg, int bh, int H, int L, int r) {
    if constexpr (!PAGED) {
        return (size_t)bh * L + r;
    } else {
        const int b = bh / H, h = bh - b * H;
        int page = pg.table[(size_t)b * pg.max_pages + (r >> pg.log2_page)];
        page = min(max(page, 0), pg.num_pages - 1);
        return (((size_t)page * H + h) << pg.log2_page) + (r & ((1 << pg.log2_page) - 1));
    }
}

// Cache length of sequence b: lens[b] clamped to [lo, L], or L without a length array.
__device__ __forceinline__ int seq_len(const int* lens, int b, int lo, int L) {
    return lens ? min(max(lens[b], lo), L) : L;
}

__device__ __forceinline__ void write_empty(float* dst, int tid) {
    if (tid == 0) {
        dst[0] = -INFINITY;
        dst[1] = 0.f;
        dst[2] = -INFINITY;
        dst[3] = 0.f;
    }
    for (int k = tid; k < 2 * DV; k += THREADS) dst[4 + k] = 0.f;
}

template <bool PAGED>
__global__ __launch_bounds__(THREADS) void decode_split_kernel(const uint16_t* __restrict__ gq1,
                                                               const uint16_t* __restrict__ gk1,
                                                               const uint16_t* __restrict__ gq2,
                                                               const uint16_t* __restrict__ gk2,
                                                               const uint16_t* __restrict__ gv,
                                                               float* __restrict__ ws, int L, int splits,
                                                               int split_keys, const int* __restrict__ lens, int H,
                                                               DecodePages pg) {
    __shared__ float sc1[MAX_SPLIT_KEYS], sc2[MAX_SPLIT_KEYS];
    __shared__ float red[4][8];
    __shared__ float part[4][2 * DV];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x / splits;
    const int sp = blockIdx.x % splits;
    const int j0 = sp * split_keys;
    const int n = min(seq_len(lens, bh / H, 1, L), j0 + split_keys) - j0;
    if (n <= 0) {   // past this sequence's end (ragged caches only)
        write_empty(ws + ((size_t)bh * splits + sp) * PART_FLOATS, tid);
        return;
    }
    const float c = LOG2E * 0.125f;  // log2(e) / sqrt(64)

    // Phase 1: scores.  Lane handles 16-byte chunk (lane % 8) of row (lane / 8) of an 8-row group; the workgroup
    // covers 32 rows per step.
    const int ch = lane & 7;
    const u32x4 qa = *(const u32x4*)(gq1 + (size_t)bh * D + ch * 8);
    const u32x4 qb = *(const u32x4*)(gq2 + (size_t)bh * D + ch * 8);
    float mx1 = -INFINITY, mx2 = -INFINITY;
    const int r_in = wave * 8 + (lane >> 3);
    for (int r0 = 0; r0 < n; r0 += 32) {
        const int r = r0 + r_in;
        const int rr = min(r, n - 1);
        const size_t kr = cache_row<PAGED>(pg, bh, H, L, j0 + rr);
        const u32x4 ka = *(const u32x4*)(gk1 + kr * D + ch * 8);
        const u32x4 kb = *(const u32x4*)(gk2 + kr * D + ch * 8);
        float s1 = dot8(qa, ka, 0.f), s2 = dot8(qb, kb, 0.f);
        s1 += __shfl_xor(s1, 1); s2 += __shfl_xor(s2, 1);
        s1 += __shfl_xor(s1, 2); s2 += __shfl_xor(s2, 2);
        s1 += __shfl_xor(s1, 4); s2 += __shfl_xor(s2, 4);
        s1 *= c;
        s2 *= c;
        if (r < n) {
            if (ch == 0) { sc1[r] = s1; sc2[r] = s2; }
            mx1 = fmaxf(mx1, s1);
            mx2 = fmaxf(mx2, s2);
        }
    }
    // Phase 2: exact split maximum and sum per map.
    mx1 = wave_max(mx1);
    mx2 = wave_max(mx2);
    if (lane == 0) { red[wave][0] = mx1; red[wave][1] = mx2; }
    __syncthreads();
    const float m1 = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
    const float m2 = fmaxf(fmaxf(red[0][1], red[1][1]), fmaxf(red[2][1], red[3][1]));
    float z1 = 0.f, z2 = 0.f;
    for (int r = tid; r < n; r += THREADS) {
        const float p1 = __builtin_amdgcn_exp2f(sc1[r] - m1);
        const float p2 = __builtin_amdgcn_exp2f(sc2[r] - m2);
        sc1[r] = p1;
        sc2[r] = p2;
        z1 += p1;
        z2 += p2;
    }
    z1 = wave_sum(z1);
    z2 = wave_sum(z2);
    if (lane == 0) { red[wave][2] = z1; red[wave][3] = z2; }
    __syncthreads();

    // Phase 3: partial outputs.  Lane handles channels 8*(lane % 16) .. +7 of row (lane / 16) of a 4-row group;
    // the workgroup covers 16 rows per step.
    const int vc = lane & 15;
    const int vr_in = wave * 4 + (lane >> 4);
    float a1[8], a2[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) { a1[k] = 0.f; a2[k] = 0.f; }
#pragma unroll 4
    for (int r0 = 0; r0 < n; r0 += 16) {
        const int r = r0 + vr_in;
        if (r < n) {
            const u32x4 w = *(const u32x4*)(gv + cache_row<PAGED>(pg, bh, H, L, j0 + r) * DV + vc * 8);
            const float p1 = sc1[r], p2 = sc2[r];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float lo = bf_lo(w[k]), hi = bf_hi(w[k]);
                a1[2 * k] = __builtin_fmaf(p1, lo, a1[2 * k]);
                a1[2 * k + 1] = __builtin_fmaf(p1, hi, a1[2 * k + 1]);
                a2[2 * k] = __builtin_fmaf(p2, lo, a2[2 * k]);
                a2[2 * k + 1] = __builtin_fmaf(p2, hi, a2[2 * k + 1]);
            }
        }
    }
    // Reduce the 4 row slots of the wave (lanes vc, vc+16, vc+32, vc+48), then the 4 waves through LDS.
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a1[k] += __shfl_xor(a1[k], 16);
        a1[k] += __shfl_xor(a1[k], 32);
        a2[k] += __shfl_xor(a2[k], 16);
        a2[k] += __shfl_xor(a2[k], 32);
    }
    if (lane < 16) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            part[wave][vc * 8 + k] = a1[k];
            part[wave][DV + vc * 8 + k] = a2[k];
        }
    }
    __syncthreads();
    float* dst = ws + ((size_t)bh * splits + sp) * PART_FLOATS;
    if (tid == 0) {
        dst[0] = m1;
        dst[1] = red[0][2] + red[1][2] + red[2][2] + red[3][2];
        dst[2] = m2;
        dst[3] = red[0][3] + red[1][3] + red[2][3] + red[3][3];
    }
    for (int k = tid; k < 2 * DV; k += THREADS) dst[4 + k] = part[0][k] + part[1][k] + part[2][k] + part[3][k];
}

// One wave per head: lane owns channels 2*lane and 2*lane + 1.
// Work item = (head, query): blockIdx.x = bh * T + t.  Every query sees at least one key, so some split is
// non-empty and the merged maxima are finite.
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ ws, uint16_t* __restrict__ gout,
                                                          int splits, int T, Epilogue ep) {
    const int item = blockIdx.x;
    const int bh = item / T;
    const int lane = threadIdx.x;
    const float* part = ws + (size_t)item * splits * PART_FLOATS;
    float M1 = -INFINITY, M2 = -INFINITY;
    for (int s = 0; s < splits; ++s) {
        M1 = fmaxf(M1, part[s * PART_FLOATS + 0]);
        M2 = fmaxf(M2, part[s * PART_FLOATS + 2]);
    }
    float L1 = 0.f, L2 = 0.f, o1a = 0.f, o1b = 0.f, o2a = 0.f, o2b = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float* p = part + s * PART_FLOATS;
        const float w1 = __builtin_amdgcn_exp2f(p[0] - M1);
        const float w2 = __builtin_amdgcn_exp2f(p[2] - M2);
        L1 += w1 * p[1];
        L2 += w2 * p[3];
        o1a += w1 * p[4 + 2 * lane];
        o1b += w1 * p[4 + 2 * lane + 1];
        o2a += w2 * p[4 + DV + 2 * lane];
        o2b += w2 * p[4 + DV + 2 * lane + 1];
    }
    const float inv1 = 1.f / L1, inv2 = lambda_of(ep, bh) / L2;
    float ya = o1a * inv1 - o2a * inv2;
    float yb = o1b * inv1 - o2b * inv2;
    if (ep.normalise) {
        const float ss = wave_sum(ya * ya + yb * yb);
        const float r = __builtin_amdgcn_rsqf(ss * (1.f / DV) + 1e-5f) * ep.out_scale;
        ya *= r;
        yb *= r;
    }
    const unsigned w = (unsigned)__builtin_bit_cast(unsigned short, (__bf16)ya) |
                       ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)yb) << 16);
    *(unsigned*)(gout + (size_t)item * DV + 2 * lane) = w;
}

// Multi-token split: one workgroup per (head, key split), all T queries of the head.
template <bool PAGED>
__global__ __launch_bounds__(THREADS) void decode_multi_split_kernel(const uint16_t* __restrict__ gq1,
                                                                     const uint16_t* __restrict__ gk1,
                                                                     const uint16_t* __restrict__ gq2,
                                                                     const uint16_t* __restrict__ gk2,
                                                                     const uint16_t* __restrict__ gv,
                                                                     float* __restrict__ ws, int L, int T, int splits,
                                                                     int split_keys, const int* __restrict__ lens,
                                                                     int H, DecodePages pg) {
    __shared__ float sc[2][MULTI_SCORES];                    // [map][t * split_keys + r]
    __shared__ __attribute__((aligned(16))) uint16_t qs[2][MAX_T][D];
    __shared__ float stat[MAX_T][4];                         // m1, l1, m2, l2 per query

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x / splits;
    const int sp = blockIdx.x % splits;
    const int Lb = seq_len(lens, bh / H, T, L);
    const int j0 = sp * split_keys;
    const int n = min(Lb, j0 + split_keys) - j0;
    const int pos0 = Lb - T;                                 // cache position of query 0
    const float c = LOG2E * 0.125f;
    float* dst0 = ws + (size_t)bh * T * splits * PART_FLOATS;
    if (n <= 0) {
        for (int t = 0; t < T; ++t) write_empty(dst0 + ((size_t)t * splits + sp) * PART_FLOATS, tid);
        return;
    }
    for (int k = tid; k < T * D / 8; k += THREADS) {        // stage the T queries (16-byte chunks)
        const int t = k / (D / 8), chunk = k % (D / 8);
        *(u32x4*)&qs[0][t][chunk * 8] = *(const u32x4*)(gq1 + ((size_t)bh * T + t) * D + chunk * 8);
        *(u32x4*)&qs[1][t][chunk * 8] = *(const u32x4*)(gq2 + ((size_t)bh * T + t) * D + chunk * 8);
    }
    __syncthreads();

    // Phase 1: scores of every query for the split's keys (masked keys -> -inf).
    const int ch = lane & 7;
    const int r_in = wave * 8 + (lane >> 3);
    for (int r0 = 0; r0 < n; r0 += 32) {
        const int r = r0 + r_in;
        const int rr = min(r, n - 1);
        const size_t kr = cache_row<PAGED>(pg, bh, H, L, j0 + rr);
        const u32x4 ka = *(const u32x4*)(gk1 + kr * D + ch * 8);
        const u32x4 kb = *(const u32x4*)(gk2 + kr * D + ch * 8);
        for (int t = 0; t < T; ++t) {
            float s1 = dot8(*(const u32x4*)&qs[0][t][ch * 8], ka, 0.f);
            float s2 = dot8(*(const u32x4*)&qs[1][t][ch * 8], kb, 0.f);
            s1 += __shfl_xor(s1, 1); s2 += __shfl_xor(s2, 1);
            s1 += __shfl_xor(s1, 2); s2 += __shfl_xor(s2, 2);
            s1 += __shfl_xor(s1, 4); s2 += __shfl_xor(s2, 4);
            if (r < n && ch == 0) {
                const bool vis = j0 + r <= pos0 + t;
                sc[0][t * split_keys + r] = vis ? s1 * c : -INFINITY;
                sc[1][t * split_keys + r] = vis ? s2 * c : -INFINITY;
            }
        }
    }
    __syncthreads();
    // Phase 2: per query (wave w takes t = w, w + 4, ...), the split's max and sum per map; probabilities in place.
    for (int t = wave; t < T; t += 4) {
        float* s1 = &sc[0][t * split_keys];
        float* s2 = &sc[1][t * split_keys];
        float m1 = -INFINITY, m2 = -INFINITY;
        for (int r = lane; r < n; r += 64) { m1 = fmaxf(m1, s1[r]); m2 = fmaxf(m2, s2[r]); }
        m1 = wave_max(m1);
        m2 = wave_max(m2);
        float z1 = 0.f, z2 = 0.f;
        if (m1 != -INFINITY) {   // the split holds at least one visible key of query t (both maps alike)
            for (int r = lane; r < n; r += 64) {
                const float p1 = __builtin_amdgcn_exp2f(s1[r] - m1), p2 = __builtin_amdgcn_exp2f(s2[r] - m2);
                s1[r] = p1;
                s2[r] = p2;
                z1 += p1;
                z2 += p2;
            }
        }
        z1 = wave_sum(z1);
        z2 = wave_sum(z2);
        if (lane == 0) {
            stat[t][0] = m1;
            stat[t][1] = z1;
            stat[t][2] = m2;
            stat[t][3] = z2;
        }
    }
    // Phase 3: partial outputs per query; lane takes channels 8 (lane % 16) .. + 7 of row slot lane / 16.
    const int vc = lane & 15, slot = lane >> 4;
    for (int t = wave; t < T; t += 4) {
        float* dst = dst0 + ((size_t)t * splits + sp) * PART_FLOATS;
        const float m1 = stat[t][0];   // written by this wave above
        float a1[8], a2[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) { a1[k] = 0.f; a2[k] = 0.f; }
        if (m1 != -INFINITY) {
            const float* p1s = &sc[0][t * split_keys];
            const float* p2s = &sc[1][t * split_keys];
            for (int r = slot; r < n; r += 4) {
                const u32x4 w = *(const u32x4*)(gv + cache_row<PAGED>(pg, bh, H, L, j0 + r) * DV + vc * 8);
                const float p1 = p1s[r], p2 = p2s[r];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float lo = bf_lo(w[k]), hi = bf_hi(w[k]);
                    a1[2 * k] = __builtin_fmaf(p1, lo, a1[2 * k]);
                    a1[2 * k + 1] = __builtin_fmaf(p1, hi, a1[2 * k + 1]);
                    a2[2 * k] = __builtin_fmaf(p2, lo, a2[2 * k]);
                    a2[2 * k + 1] = __builtin_fmaf(p2, hi, a2[2 * k + 1]);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            a1[k] += __shfl_xor(a1[k], 16);
            a1[k] += __shfl_xor(a1[k], 32);
            a2[k] += __shfl_xor(a2[k], 16);
            a2[k] += __shfl_xor(a2[k], 32);
        }
        if (lane < 16) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                dst[4 + vc * 8 + k] = a1[k];
                dst[4 + DV + vc * 8 + k] = a2[k];
            }
        }
        if (lane == 0) {
            dst[0] = stat[t][0];
            dst[1] = stat[t][1];
            dst[2] = stat[t][2];
            dst[3] = stat[t][3];
        }
    }
}

// Split plan of a call: the single-token plan, with splits shortened for T > 1 so that T x split keys fit in LDS.
SplitPlan plan_call(int64_t BH, int64_t L, int T) {
    SplitPlan p = plan_splits(BH, L);
    if (T > 1) {
        int cap = (MULTI_SCORES / T) & ~31;
        if (p.split_keys > cap) {
            p.split_keys = cap;
            p.splits = (int)((L + cap - 1) / cap);
        }
    }
    return p;
}

}  // namespace

size_t decode_bf16_workspace_bytes(int64_t BH, int64_t L, int T) {
    if (BH <= 0 || L <= 0 || T < 1 || T > MAX_T) return 0;
    const SplitPlan p = plan_call(BH, L, T);
    return (size_t)BH * (size_t)T * (size_t)p.splits * PART_FLOATS * sizeof(float);
}

hipError_t launch_decode_bf16_d64(const uint16_t* q1, const uint16_t* k1, const uint16_t* q2, const uint16_t* k2,
                                  const uint16_t* v, uint16_t* out, int64_t BH, int64_t H, int64_t L, int T,
                                  const int* lens, const DecodePages* pages, Epilogue ep, void* workspace,
                                  hipStream_t stream) {
    const SplitPlan p = plan_call(BH, L, T);
    const int64_t blocks = BH * (int64_t)p.splits;
    if (blocks > 0x7fffffff || BH * T > 0x7fffffff || T < 1 || T > MAX_T) return hipErrorInvalidValue;
    if (pages && ((int64_t)pages->max_pages << pages->log2_page) != L) return hipErrorInvalidValue;
    float* ws = (float*)workspace;
    const DecodePages pg = pages ? *pages : DecodePages{nullptr, 0, 0, 0};
    if (T == 1) {
        if (pages)
            hipLaunchKernelGGL(decode_split_kernel<true>, dim3((unsigned)blocks), dim3(THREADS), 0, stream, q1, k1, q2,
                               k2, v, ws, (int)L, p.splits, p.split_keys, lens, (int)H, pg);
        else
            hipLaunchKernelGGL(decode_split_kernel<false>, dim3((unsigned)blocks), dim3(THREADS), 0, stream, q1, k1,
                               q2, k2, v, ws, (int)L, p.splits, p.split_keys, lens, (int)H, pg);
    } else {
        if (pages)
            hipLaunchKernelGGL(decode_multi_split_kernel<true>, dim3((unsigned)blocks), dim3(THREADS), 0, stream, q1,
                               k1, q2, k2, v, ws, (int)L, T, p.splits, p.split_keys, lens, (int)H, pg);
        else
            hipLaunchKernelGGL(decode_multi_split_kernel<false>, dim3((unsigned)blocks), dim3(THREADS), 0, stream, q1,
                               k1, q2, k2, v, ws, (int)L, T, p.splits, p.split_keys, lens, (int)H, pg);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(BH * T)), dim3(64), 0, stream, (const float*)ws, out,
                       p.splits, T, ep);
    return hipGetLastError();
}

}  // namespace diffattn
