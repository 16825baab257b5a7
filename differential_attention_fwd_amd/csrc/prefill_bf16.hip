// Fused one-pass differential attention prefill for gfx950 (bf16 in/out, fp32 accumulation, d = 64, 2d = 128).
//
// Operation (Ultralytics glossary "Differential Transformer", section on how differential attention works: worked
// example and the paragraph after it): per head and query row i, two softmax maps over the visible keys with
// scores q1.k1/sqrt(d) and q2.k2/sqrt(d), output sum_j (a_j - lambda b_j) v_j, then optionally the per-head RMS
// normalisation and the (1 - lambda_init) scale.
//
// Design (one pass over K1/K2/V, nothing N x N ever materialised):
//   * A workgroup of 4 waves (one per SIMD) owns 128 query rows of one (batch, head); each wave owns 32 rows.  Two
//     workgroups share a CU, so each SIMD runs two independent waves and the matrix cores of one overlap the
//     softmax of the other.  Key tiles are 32 keys.
//   * Loads go straight from global memory to LDS (buffer_load ... lds, no registers) through 4-slot rings, three
//     tiles ahead: K1, K2 and V tiles, laid out in LDS so that every operand read is free of bank conflicts.
//     Ring slots are separate __shared__ arrays and the loop is unrolled by four, so the compiler can tell reads
//     of one slot from loads still landing in another.  One workgroup barrier per tile.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in
//     registers).  In the accumulator layout every lane owns ONE query row (lane % 32) and 16 of the 32 keys, so
//     row statistics need only the lane pair (l, l ^ 32), exchanged with v_permlane32_swap.
//   * P^T stays in registers and feeds O^T = V^T P^T directly as the MFMA B operand.  The k-order of that product
//     is the accumulator's key order.  The A operand (V^T: one channel, 8 keys per lane) comes from the
//     key-by-key V tile through two transposing reads (ds_read_b64_tr_b16, 4 keys each) that pick the keys in that order;
//     each fragment is shared by the two maps.  O^T's layout gives each lane one query row again, so the
//     online-softmax rescale of O is lane-local.
//   * Two online softmaxes run side by side (running offset and sum per map, two O accumulators).  Probabilities
//     are taken at the running offset first; only when a lane's 16 of them sum to more than 2^8 (a wave-uniform
//     decision) is the row max taken and O rescaled, so neither the max nor the rescale is on the common path.
//     Exponents use exp2 with log2(e)/sqrt(d) folded into one FMA; the row sums add the probabilities in fp32 with
//     plain VALU adds (v_dot2 would run on the matrix pipe and wait behind the MFMAs).  Map 2's exponentials are
//     issued between map 1's value MFMAs.
//   * Epilogue: O1/l1 - lambda O2/l2, RMS over the 128 channels (pair-reduced), scale, bf16 round-to-nearest-even.
//   * Causal: row tiles are launched heaviest first; tiles wholly above a wave's rows are skipped by that wave,
//     and only diagonal or ragged-tail tiles pay for masking.  Each XCD takes its heads a few at a time (xcd_item),
//     so that fewer heads' K and V compete for its L2.
//
// This translation unit is compiled with -fno-honor-nans: no NaN can arise (inputs are finite, masked scores are
// -inf, the running offsets start at -FLT_MAX rather than -inf, and every processed row has a visible key in its
// first tile), and it lets v_max3 run without quieting.
#include <algorithm>
#include <mutex>

#include "launch.h"
#include "tiles.h"

namespace diffattn {
namespace {

constexpr int D = 64;
constexpr int DV = 128;
constexpr int WAVES = 4;                        // waves per workgroup, 32 query rows each
constexpr int BM = 32 * WAVES;                  // query rows per workgroup
constexpr int BN = 32;                          // keys per tile
constexpr int THREADS = 64 * WAVES;
constexpr int K_TILE_BYTES = BN * D * 2;        // 4 KiB
constexpr int V_TILE_BYTES = BN * DV * 2;       // 8 KiB
constexpr int RING = 4;                         // ring slots: K and V tiles t in slot t % 4, loaded three ahead
constexpr int K_SLOT_BYTES = 2 * K_TILE_BYTES;

// Compile-time ring slot.  Each ring slot is its own __shared__ array, so the compiler can tell an LDS read of one
// slot from a direct load still landing in another and does not drain the prefetches before every LDS read.
template <int V> struct Slot { static constexpr int value = V; };
template <bool V> struct Flag { static constexpr bool value = V; };
template <int S, class T> __device__ __forceinline__ T* pick4(T* a, T* b, T* c, T* d) {
    static_assert(RING == 4, "one array per ring slot");
    if constexpr (S % 4 == 0) return a;
    else if constexpr (S % 4 == 1) return b;
    else if constexpr (S % 4 == 2) return c;
    else return d;
}
// A lane's 16 probabilities of a tile may sum to at most 2^8 at the running offset; above that (or +inf) the tile takes
// the exact path.  So no probability ever exceeds 2^8 between rescales.
constexpr unsigned P_SUM_LIMIT_BITS = 0x43800000u;   // bits of 256.0f; compared as integers, +inf and NaN exceed it

__device__ __forceinline__ float max16(const f32x16& s) {
    const float a = fmaxf(fmaxf(s[0], s[1]), s[2]), b = fmaxf(fmaxf(s[3], s[4]), s[5]);
    const float c = fmaxf(fmaxf(s[6], s[7]), s[8]), d = fmaxf(fmaxf(s[9], s[10]), s[11]);
    const float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
    return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), s[15]));
}

// Online-softmax state of one map for the lane's query row: the running offset in score units (ms) and in log2
// units (ml = ms * c), and the running sum l.  Both offsets start at -FLT_MAX, so the first tile's probabilities
// overflow to +inf (never NaN, also for masked -inf scores) and take the exact path.
struct MapState {
    float ms, ml, l;
};

// p = exp2(s * c - ml) for the lane's 16 keys, packed as P^T: two bf16x8 B operands.  Returns the sum of the 16
// probabilities in fp32.
__device__ __forceinline__ float exp_pack(const f32x16& s, float ml, float c, bf16x8& lo, bf16x8& hi) {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -ml));
    u32x4 a, b;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        a[k] = pack2(p[2 * k], p[2 * k + 1]);
        b[k] = pack2(p[8 + 2 * k], p[8 + 2 * k + 1]);
    }
    lo = __builtin_bit_cast(bf16x8, a);
    hi = __builtin_bit_cast(bf16x8, b);
    float t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = p[2 * k] + p[2 * k + 1];
    return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

// Probabilities of one map for the lane's 16 scores of a tile, packed as P^T (lo, hi), and their sum.  They are
// first taken at the running offset.  Only if some lane's sum exceeds 2^8 (a wave-uniform decision; the first tile
// always does) is the row max taken: the offset moves to it, O and l are rescaled, and the probabilities are taken
// again.  Between rescales every probability is at most 2^8, and after the first few tiles the row max is almost
// never needed.
__device__ __forceinline__ float softmax_tile(const f32x16& s, MapState& st, f32x16 (&o)[4], float c, bf16x8& lo,
                                              bf16x8& hi) {
    float part = exp_pack(s, st.ml, c, lo, hi);
    if (__any(__float_as_uint(part) > P_SUM_LIMIT_BITS)) {
        const float ms = fmaxf(st.ms, pair_max(max16(s)));
        const float ml = ms * c;
        const float alpha = __builtin_amdgcn_exp2f(st.ml - ml);
        st.ms = ms;
        st.ml = ml;
        st.l *= alpha;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
        part = exp_pack(s, ml, c, lo, hi);
    }
    return part;
}

// The first tile of a wave's rows (every row sees at least one of its keys): the offset is the tile's row max, and O
// and l are still zero, so nothing is rescaled.  Same values as softmax_tile's exact path from the initial state.
__device__ __forceinline__ float softmax_first(const f32x16& s, MapState& st, float c, bf16x8& lo, bf16x8& hi) {
    st.ms = pair_max(max16(s));
    st.ml = st.ms * c;
    return exp_pack(s, st.ml, c, lo, hi);
}

// Key-split launches: the key tiles of a row tile are cut into ranges of kt_split tiles; a causal row tile reaches
// only the ranges up to its diagonal, so it has fewer.  One workgroup per non-empty (row tile, head, range) item,
// which writes each row's partial state for its range (PARTIAL_FLOATS in launch.h, row-major over (b, h, row, split))
// instead of the output.  The grid holds no empty item, and items are ordered by the number of ranges their row tile
// has, most first (the causal diagonal's and the last tile's being the longest runs), so that consecutive workgroups,
// which the hardware deals out to the XCDs in turn, are alike in cost.
struct KeySplit {
    int splits, kt_split;
    float* part;
};

// The first row tile of a causal launch that reaches range j - 1, i.e. has at least j ranges (j >= 1): row tile rt
// < n_row_tiles - 1 spans (rt + 1) BM / BN key tiles, the last one all of them.
__device__ __host__ inline int first_row_tile_with(int j, int kt_split, int n_row_tiles) {
    const int64_t r = (int64_t)(j - 1) * kt_split * BN / BM;
    return r < n_row_tiles - 1 ? (int)r : n_row_tiles - 1;
}

// Number of ranges of causal row tile rt.
__device__ __host__ inline int ranges_of(int rt, int kt_split, int n_row_tiles, int key_tiles) {
    const int kend = rt == n_row_tiles - 1 ? key_tiles : (rt + 1) * (BM / BN);
    return (kend + kt_split - 1) / kt_split;
}

// SAVE: also write each row's training statistics (SAVED_* in launch.h) for the backward pass.
// SPLIT: cover one key range of the row tile and write partial states (KeySplit).
// xcd_group: without SPLIT, the heads each XCD takes at a time (xcd_item in launch.h; 0: all of them).
template <bool SAVE, bool SPLIT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_d64_kernel(const uint16_t* __restrict__ gq1, const uint16_t* __restrict__ gk1,
                             const uint16_t* __restrict__ gq2, const uint16_t* __restrict__ gk2,
                             const uint16_t* __restrict__ gv, uint16_t* __restrict__ gout, int BH, int H, int N,
                             int n_row_tiles, int causal, Strides st, Epilogue ep, float* __restrict__ saved,
                             KeySplit ks, int xcd_group) {
    __shared__ __attribute__((aligned(16))) unsigned char kr0[K_SLOT_BYTES], kr1[K_SLOT_BYTES], kr2[K_SLOT_BYTES],
        kr3[K_SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char vr0[V_TILE_BYTES], vr1[V_TILE_BYTES], vr2[V_TILE_BYTES],
        vr3[V_TILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int h = lane >> 5;     // which half of the accumulator's key rows this lane holds
    const int l32 = lane & 31;   // this lane's query row inside the wave

    // Heaviest row tiles first under the causal mask (their key range is longest).
    int rt, bh, sp = 0;
    if constexpr (SPLIT) {
        // Groups of row tiles with j ranges, j = splits down to 1; inside a group row tiles descend, then heads,
        // then ranges.  Every launched workgroup falls in some group (the host sized the grid as their sum).
        int rem = (int)blockIdx.x, j = ks.splits, hi = n_row_tiles;
        if (causal) {
            for (; j > 1; --j) {
                const int lo = first_row_tile_with(j, ks.kt_split, n_row_tiles);
                const int cnt = (hi - lo) * BH * j;
                if (rem < cnt) break;
                rem -= cnt;
                hi = lo;
            }
        }
        rt = hi - 1 - rem / (BH * j);
        bh = rem % (BH * j) / j;
        sp = rem % j;
    } else {
        int r;
        xcd_item((int)blockIdx.x, BH, n_row_tiles, xcd_group, r, bh);
        rt = causal ? (n_row_tiles - 1 - r) : r;
    }
    const int q0 = rt * BM;
    const int q0w = q0 + wave * 32;

    // This head's first element in each tensor (strides in elements; the feature dimension is contiguous).
    const int64_t b_ = bh / H, h_ = bh % H;
    auto base = [&](int k) { return b_ * st.b[k] + h_ * st.h[k]; };
    // Per-head buffer resources over the head's N rows: rows at or beyond N read as zero (and are masked), so no
    // clamping is needed.  Offsets are unsigned 32-bit; the host checked that N + 256 rows fit.
    const unsigned k1rb = (unsigned)st.n[S_K1] * 2u, k2rb = (unsigned)st.n[S_K2] * 2u, vrb = (unsigned)st.n[S_V] * 2u;
    const unsigned n1 = (unsigned)(N - 1);
    const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc((void*)(gk1 + base(S_K1)), (short)0,
                                                                         (int)(n1 * k1rb + D * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rk2 = __builtin_amdgcn_make_buffer_rsrc((void*)(gk2 + base(S_K2)), (short)0,
                                                                         (int)(n1 * k2rb + D * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(gv + base(S_V)), (short)0,
                                                                        (int)(n1 * vrb + DV * 2u), 0x00020000);

    // Q fragments as the MFMA B operand: lane holds Q[q0w + l32][16 kc + 8 h .. + 7].
    bf16x8 qa[4], qb[4];
    {
        const int row = min(q0w + l32, N - 1);
        const uint16_t* p1 = gq1 + base(S_Q1) + (int64_t)row * st.n[S_Q1] + 8 * h;
        const uint16_t* p2 = gq2 + base(S_Q2) + (int64_t)row * st.n[S_Q2] + 8 * h;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            qa[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(p1 + 16 * kc));
            qb[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(p2 + 16 * kc));
        }
    }

    const int q_last = min(N, q0 + BM) - 1;
    const int n_tiles = causal ? (q_last / BN + 1) : (N + BN - 1) / BN;
    // Key tiles of this workgroup: all of the row tile's, or one split's share.
    const int kt0 = SPLIT ? sp * ks.kt_split : 0;
    const int kt_end = SPLIT ? min(n_tiles, kt0 + ks.kt_split) : n_tiles;
    // Direct loads: each wave moves one 1 KiB piece per tile and tensor role.  K1 and K2 tiles (4 KiB each) are 8
    // pieces, the V tile (8 KiB) another 8; piece x of a tile covers its bytes [1024 x, 1024 x + 1024) and lane L
    // writes position 16 L of it.  Loads are issued unconditionally, also for tiles past the end: those buffer loads
    // are out of range and read zeros, and they land in ring slots no wave reads again.  The number of vector-memory
    // operations per iteration is therefore fixed, which makes the waits below exact.
    constexpr int K_PIECES_PER_WAVE = 8 / WAVES;   // K1 + K2 pieces per wave and tile
    constexpr int V_PIECES_PER_WAVE = 8 / WAVES;
    unsigned kd_voff[K_PIECES_PER_WAVE], kd_step[K_PIECES_PER_WAVE], vd_voff[V_PIECES_PER_WAVE];
    int kd_lds[K_PIECES_PER_WAVE];
#pragma unroll
    for (int j = 0; j < K_PIECES_PER_WAVE; ++j) {
        const int piece = wave + WAVES * j;        // 0..3: K1, 4..7: K2
        const unsigned rb = piece < 4 ? k1rb : k2rb;
        // Piece kc = piece % 4 of a K tile holds 16-byte chunks 2 kc and 2 kc + 1 of all 32 rows: chunk 2 kc + e of
        // row r at position 2 r + (e ^ ((r >> 3) & 1)), so lane L brings row L / 2, chunk 2 kc + ((L & 1) ^ ...).
        const int row = lane >> 1, kc = piece & 3;
        kd_voff[j] = (unsigned)row * rb + ((2 * kc + ((lane & 1) ^ ((row >> 3) & 1))) << 4);
        kd_step[j] = (unsigned)BN * rb;            // bytes per tile
        kd_lds[j] = (piece >> 2) * K_TILE_BYTES + 1024 * (piece & 3);
    }
#pragma unroll
    for (int j = 0; j < V_PIECES_PER_WAVE; ++j) {
        // V tile as [channel block][key][32 channels] (2 KiB per block of 32 channels): piece x holds channels
        // 32 (x / 2) .. + 31 of keys 16 (x % 2) .. + 15, 64 bytes per key, so lane L brings key 16 (x % 2) + L / 4,
        // bytes 16 (L % 4) .. + 15 of that channel block.
        const int x = wave + WAVES * j;
        const int row = 16 * (x & 1) + (lane >> 2);
        vd_voff[j] = (unsigned)row * vrb + 64 * (x >> 1) + 16 * (lane & 3);
    }
    const unsigned vd_step = (unsigned)BN * vrb;
    auto issue_k = [&](auto S, int t) {   // S = t % 4
        unsigned char* slot = pick4<decltype(S)::value>(kr0, kr1, kr2, kr3);
#pragma unroll
        for (int j = 0; j < K_PIECES_PER_WAVE; ++j) check_fill(slot + kd_lds[j], 16);
        check_fence();
#pragma unroll
        for (int j = 0; j < K_PIECES_PER_WAVE; ++j) {
            // The tile offset goes into the VGPR offset: the SGPR offset is not part of the buffer range check.
            const unsigned ko = kd_voff[j] + (unsigned)t * kd_step[j];
            if ((wave + WAVES * j) < 4)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk1, (lds_void*)(slot + kd_lds[j]), 16, (int)ko, 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk2, (lds_void*)(slot + kd_lds[j]), 16, (int)ko, 0, 0, 0);
        }
    };
    auto issue_v = [&](auto S, int t) {   // S = t % 4
        unsigned char* slot = pick4<decltype(S)::value>(vr0, vr1, vr2, vr3);
#pragma unroll
        for (int j = 0; j < V_PIECES_PER_WAVE; ++j) check_fill(slot + 1024 * (wave + WAVES * j), 16);
        check_fence();
#pragma unroll
        for (int j = 0; j < V_PIECES_PER_WAVE; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(slot + 1024 * (wave + WAVES * j)), 16,
                                                     (int)(vd_voff[j] + (unsigned)t * vd_step), 0, 0, 0);
    };
    // Per-lane read offsets.  The LDS serves a 128-bit read in four windows of 16 lanes (within each half wave, the
    // 4-lane groups (lane >> 2) & 7 of even and of odd bit parity) and a 64-bit read in two windows of 32
    // consecutive lanes; both layouts give every window distinct banks, and every fragment a constant offset.
    // K A-operand: row l32, chunk 2 kc + h, at 1024 kc + 16 (2 l32 + (h ^ ((l32 >> 3) & 1))).
    // V^T A-operand of channel block cb and key half ks: lane (h, l32) needs channel 32 cb + l32 of the keys at
    // accumulator positions 16 ks + 8 h .. + 7, i.e. keys 16 ks + 4 h + 0..3, then 16 ks + 8 + 4 h + 0..3.  Each
    // comes from one ds_read_b64_tr_b16: the lane's 16-lane group reads a block of 4 keys x 16 channels, lane
    // 4 jj + q of the group supplying key jj, channels 4 q .. 4 q + 3 of the block, and lane i of the group
    // receiving channel i of the 4 keys.  A 32-lane window reads 4 whole 64-byte key rows of a channel block
    // (256 contiguous bytes); channel block cb adds 2 KiB, 16 keys 1 KiB, 8 keys 512 bytes.
    const int k_rd0 = 16 * (2 * l32 + (h ^ ((l32 >> 3) & 1)));
    const int trl = lane & 15;
    const int tr_ch = 16 * ((lane >> 4) & 1) + 4 * (trl & 3);   // first channel this lane supplies (block cb = 0)
    const int v_rd0 = 64 * (4 * h + (trl >> 2)) + 2 * tr_ch;

    f32x16 o1[4], o2[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) { o1[cb][i] = 0.f; o2[cb][i] = 0.f; }
    const float c = LOG2E * 0.125f;  // log2(e) / sqrt(64)
    MapState st1 = {-__FLT_MAX__, -__FLT_MAX__, 0.f}, st2 = st1;

    // Load schedule.  Iteration t (between two workgroup barriers) issues the direct loads of K(t + 3) and V(t + 3)
    // into the slot that tile t - 1 left (every wave has passed the barrier after reading it), and computes tile t.
    // At its end it waits for everything but the loads of this iteration and the previous one, so tile t + 1 has
    // landed and a load has two whole iterations to land.
    issue_k(Slot<0>{}, kt0);
    issue_v(Slot<0>{}, kt0);
    issue_k(Slot<1>{}, kt0 + 1);
    issue_v(Slot<1>{}, kt0 + 1);
    issue_k(Slot<2>{}, kt0 + 2);
    issue_v(Slot<2>{}, kt0 + 2);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * (K_PIECES_PER_WAVE + V_PIECES_PER_WAVE)));
    lds_barrier();
    // Two transposing reads make one V^T fragment (the 8 keys of one accumulator position block).
    auto v_frag = [&](const unsigned char* p) __attribute__((always_inline)) {
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * 64));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // Mask bound of tile kv0: key kv0 + 8 (i / 4) + 4 h + i % 4 is visible to the lane's row q iff it is at most
    // min(q, N - 1), i.e. iff 8 (i / 4) + i % 4 <= min(q, N - 1) - kv0 - 4 h (compile-time left-hand sides).
    const int q_vis = min(q0w + l32, N - 1) - 4 * h;
    auto step = [&](auto S, auto FIRST, int t) {   // S = t % 4; FIRST: the wave's first tile (t = 0)
        constexpr int s0 = decltype(S)::value;
        constexpr bool first = decltype(FIRST)::value;
        issue_k(Slot<(s0 + 3) % 4>{}, t + 3);
        issue_v(Slot<(s0 + 3) % 4>{}, t + 3);
        const int kv0 = t * BN;
        if (!causal || kv0 <= q0w + 31) {
            const unsigned char* kb_ = pick4<s0>(kr0, kr1, kr2, kr3);
            const unsigned char* vb_ = pick4<s0>(vr0, vr1, vr2, vr3);
            // Wave priority: high while this wave issues matrix work, low for map 1's softmax, so that of the two
            // waves on a SIMD the one with MFMAs ready wins the issue arbitration.
            __builtin_amdgcn_s_setprio(1);
            f32x16 s1, s2;
#pragma unroll
            for (int i = 0; i < 16; ++i) { s1[i] = 0.f; s2[i] = 0.f; }
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const int kro = k_rd0 + 1024 * kc;
                const bf16x8 ka = *(const bf16x8*)(kb_ + kro);
                const bf16x8 kb = *(const bf16x8*)(kb_ + K_TILE_BYTES + kro);
                s1 = mfma(ka, qa[kc], s1);
                s2 = mfma(kb, qb[kc], s2);
            }
            if ((causal && kv0 + BN - 1 > q0w) || kv0 + BN > N) {
                const int d = (causal ? q_vis : N - 1 - 4 * h) - kv0;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const bool vis = 8 * (i >> 2) + (i & 3) <= d;
                    s1[i] = vis ? s1[i] : -INFINITY;
                    s2[i] = vis ? s2[i] : -INFINITY;
                }
            }
            bf16x8 p1[2], p2[2];
            __builtin_amdgcn_s_setprio(0);
            const float part1 = first ? softmax_first(s1, st1, c, p1[0], p1[1]) : softmax_tile(s1, st1, o1, c, p1[0], p1[1]);
            __builtin_amdgcn_s_setprio(1);
            bf16x8 va[4][2];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) va[cb][0] = v_frag(vb_ + v_rd0 + 2048 * cb);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o1[cb] = mfma(va[cb][0], p1[0], o1[cb]);
            const float part2 = first ? softmax_first(s2, st2, c, p2[0], p2[1]) : softmax_tile(s2, st2, o2, c, p2[0], p2[1]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) va[cb][1] = v_frag(vb_ + v_rd0 + 2048 * cb + 1024);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o2[cb] = mfma(va[cb][0], p2[0], o2[cb]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o1[cb] = mfma(va[cb][1], p1[1], o1[cb]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o2[cb] = mfma(va[cb][1], p2[1], o2[cb]);
            st1.l += part1;
            st2.l += part2;
            __builtin_amdgcn_s_setprio(0);
        }
        // The loads of this iteration and the previous one (tiles t + 3 and t + 2) may stay in flight past the
        // barrier; tile t + 1 has landed.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * (K_PIECES_PER_WAVE + V_PIECES_PER_WAVE)));
        lds_barrier();
    };
    // A split's first tile may hide every key from some rows, so it takes the general path (which keeps such rows'
    // states empty without NaN); a whole row tile's first tile shows every row its first key.
    step(Slot<0>{}, Flag<!SPLIT>{}, kt0);
    for (int t = kt0 + 1; t < kt_end; t += 4) {
        step(Slot<1>{}, Flag<false>{}, t);
        if (t + 1 < kt_end) step(Slot<2>{}, Flag<false>{}, t + 1);
        if (t + 2 < kt_end) step(Slot<3>{}, Flag<false>{}, t + 2);
        if (t + 3 < kt_end) step(Slot<0>{}, Flag<false>{}, t + 3);
    }
    // Drain the trailing prefetches before the workgroup can retire (their LDS writes must not outlive it).
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

    if constexpr (SPLIT) {
        // Partial state of each row for this key range: offsets (log2 units of the scaled scores), sums at those
        // offsets (l = 0 and offset -inf for a row that saw no key here), unnormalised O1 and O2.
        const float l1 = pair_sum(st1.l), l2 = pair_sum(st2.l);
        const int q = q0w + l32;
        if (q < N) {
            float* dst = ks.part + ((size_t)bh * N + q) * ks.splits * PARTIAL_FLOATS + (size_t)sp * PARTIAL_FLOATS;
            if (h == 0)
                *(f32x4*)dst = f32x4{l1 > 0.f ? st1.ml : -INFINITY, l1, l2 > 0.f ? st2.ml : -INFINITY, l2};
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int ch = cb * 32 + 8 * g4 + 4 * h;
                    *(f32x4*)(dst + 4 + ch) = f32x4{o1[cb][4 * g4], o1[cb][4 * g4 + 1], o1[cb][4 * g4 + 2],
                                                    o1[cb][4 * g4 + 3]};
                    *(f32x4*)(dst + 4 + DV + ch) = f32x4{o2[cb][4 * g4], o2[cb][4 * g4 + 1], o2[cb][4 * g4 + 2],
                                                         o2[cb][4 * g4 + 3]};
                }
        }
        return;
    }

    // Epilogue: lane owns query row q0w + l32 and channels cb*32 + 8*(i/4) + 4h + i%4.
    const float l1 = pair_sum(st1.l);
    const float l2 = pair_sum(st2.l);
    const float inv1 = 1.f / l1;
    const float inv2 = lambda_of(ep, bh) / l2;
    const int q = q0w + l32;
    float* srow = nullptr;
    if constexpr (SAVE) {
        // The two maps' normalised outputs, O1 / l1 and O2 / l2, before they are combined.
        if (q < N) {
            srow = saved + ((size_t)bh * N + q) * SAVED_FLOATS;
            const float r2 = 1.f / l2;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int ch = cb * 32 + 8 * g4 + 4 * h;
                    f32x4 a, b;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] = o1[cb][4 * g4 + e] * inv1;
                        b[e] = o2[cb][4 * g4 + e] * r2;
                    }
                    *(f32x4*)(srow + SAVED_O1 + ch) = a;
                    *(f32x4*)(srow + SAVED_O2 + ch) = b;
                }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            // One explicit fused multiply-add over a rounded product: the training variant, which also stores
            // o1 * inv1, then produces the same output bits (contraction could otherwise fuse either product).
            const float t2 = o2[cb][i] * inv2;
            const float o = __builtin_fmaf(o1[cb][i], inv1, -t2);
            o1[cb][i] = o;
            ss += o * o;
        }
    float rr = 1.f;   // 1 / sqrt(mean(o^2) + eps) when normalising
    if (ep.normalise) {
        ss = pair_sum(ss);
        rr = __builtin_amdgcn_rsqf(ss * (1.f / DV) + 1e-5f);
    }
    const float r = ep.normalise ? rr * ep.out_scale : 1.f;
    if constexpr (SAVE) {
        // Log-sum-exp of each map in log2 units of the scaled scores: p = 2^(s * log2(e) / sqrt(d) - lse).
        if (q < N && h == 0)
            *(f32x4*)srow = f32x4{st1.ml + __builtin_amdgcn_logf(l1), st2.ml + __builtin_amdgcn_logf(l2), rr, 0.f};
    }
    if (q < N) {
        uint16_t* orow = gout + base(S_OUT) + (int64_t)q * st.n[S_OUT] + 4 * h;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                u32x2 w;
                w[0] = pack2(o1[cb][4 * g4 + 0] * r, o1[cb][4 * g4 + 1] * r);
                w[1] = pack2(o1[cb][4 * g4 + 2] * r, o1[cb][4 * g4 + 3] * r);
                *(u32x2*)(orow + cb * 32 + 8 * g4) = w;
            }
    }
}

// One wave per query row, four rows per workgroup: the row's non-empty ranges merged (merge_partial_row) into the
// dense [BH][N][DV] output.
__global__ __launch_bounds__(256) void prefill_merge_kernel(const float* __restrict__ part, uint16_t* __restrict__ out,
                                                            int BH, int N, int causal, int splits, int kt_split,
                                                            int n_row_tiles, Epilogue ep) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (int64_t)BH * N) return;
    const int q = (int)(row % N);
    const int n = causal ? ranges_of(q / BM, kt_split, n_row_tiles, (N + BN - 1) / BN) : splits;
    merge_partial_row(part + row * splits * PARTIAL_FLOATS, n, ep, (int)(row / N), out + row * DV,
                      (int)(threadIdx.x & 63));
}

// Workgroups of a split launch: the non-empty (row tile, head, range) items, counted by group as the kernel walks
// them.
int64_t split_items(int64_t BH, int n_row_tiles, int splits, int kt_split, int causal) {
    if (!causal) return (int64_t)n_row_tiles * BH * splits;
    int64_t n = 0;
    int hi = n_row_tiles;
    for (int j = splits; j >= 1; --j) {
        const int lo = j > 1 ? first_row_tile_with(j, kt_split, n_row_tiles) : 0;
        n += (int64_t)(hi - lo) * BH * j;
        hi = lo;
    }
    return n;
}

}  // namespace

namespace {

// Modelled end of one XCD's schedule (see xcd_head_group in launch.h).
double xcd_makespan(int heads, int R, int causal, double fixed, int group, int slots) {
    constexpr int SLOTS_MAX = 256;
    const int ns = slots < 1 ? 1 : slots > SLOTS_MAX ? SLOTS_MAX : slots;
    double slot[SLOTS_MAX] = {};
    const auto later = [](double a, double b) { return a > b; };
    double end = 0.0;
    for (int q = 0; q < heads / group; ++q)
        for (int r = 0; r < R; ++r) {
            const double cost = fixed + (causal ? R - r : R);
            for (int hj = 0; hj < group; ++hj) {
                std::pop_heap(slot, slot + ns, later);
                slot[ns - 1] += cost;
                end = fmax(end, slot[ns - 1]);
                std::push_heap(slot, slot + ns, later);
            }
        }
    return end;
}

}  // namespace

// At B4 H12 N4096 the prefill's six heads per XCD read K and V from beyond the L2 2.0 times over (297 MB per launch
// against 151 MB of inputs); three heads at a time: 197 MB, time-neutral; two heads (modelled 19% longer): 5% slower.
int xcd_head_group(int64_t BH, int64_t R, int causal, double fixed_units, int slots) {
    if (BH <= 0 || R <= 0 || (BH & 7) != 0) return 0;
    const int64_t heads = BH / 8;
    if (heads * R > (1 << 16)) return 0;   // the model's cost grows with the items; such launches keep the plain order
    struct Plan {
        int64_t BH, R;
        int causal;
        double fixed;
        int slots, group;
    };
    static std::mutex mu;
    static Plan kept[16];
    static int kept_n = 0, next = 0;
    causal = causal ? 1 : 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < kept_n; ++i)
            if (kept[i].BH == BH && kept[i].R == R && kept[i].causal == causal && kept[i].fixed == fixed_units &&
                kept[i].slots == slots)
                return kept[i].group;
    }
    const double plain = xcd_makespan((int)heads, (int)R, causal, fixed_units, (int)heads, slots);
    int group = 0;
    for (int g = 1; g < heads; ++g)
        if (heads % g == 0 && xcd_makespan((int)heads, (int)R, causal, fixed_units, g, slots) <= 1.005 * plain) {
            group = g;
            break;
        }
    std::lock_guard<std::mutex> lock(mu);
    kept[next] = Plan{BH, R, causal, fixed_units, slots, group};
    next = (next + 1) % 16;
    kept_n = kept_n < 16 ? kept_n + 1 : 16;
    return group;
}

hipError_t launch_prefill_bf16_d64(const uint16_t* q1, const uint16_t* k1, const uint16_t* q2, const uint16_t* k2,
                                   const uint16_t* v, uint16_t* out, int64_t B, int64_t H, int64_t N, int causal,
                                   const Strides& st, Epilogue ep, float* saved, hipStream_t stream) {
    const int64_t BH = B * H;
    const int n_row_tiles = (int)((N + BM - 1) / BM);
    const int64_t blocks = (int64_t)n_row_tiles * BH;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const KeySplit none{1, 0, nullptr};
    // A row tile's fixed cost (prologue, diagonal tiles, epilogue: 14.0 K cycles) in units of the 4 key tiles
    // (4 x 2262 cycles) by which consecutive row tiles differ.
    const int xg = xcd_head_group(BH, n_row_tiles, causal, 14000.0 / (4 * 2262.0), 64);   // two workgroups per CU
    if (saved)
        hipLaunchKernelGGL((prefill_bf16_d64_kernel<true, false>), dim3((unsigned)blocks), dim3(THREADS), 0, stream,
                           q1, k1, q2, k2, v, out, (int)BH, (int)H, (int)N, n_row_tiles, causal ? 1 : 0, st, ep, saved,
                           none, xg);
    else
        hipLaunchKernelGGL((prefill_bf16_d64_kernel<false, false>), dim3((unsigned)blocks), dim3(THREADS), 0, stream,
                           q1, k1, q2, k2, v, out, (int)BH, (int)H, (int)N, n_row_tiles, causal ? 1 : 0, st, ep, saved,
                           none, xg);
    return hipGetLastError();
}

namespace {

constexpr int SPLIT_SLOTS = 512;        // workgroup slots of the GPU for this kernel: two per CU, 256 CUs
constexpr int SPLIT_MAX_ITEMS = 1024;   // plans with more items than this are not considered

// Modelled time (us) of a split launch with s ranges of kt key tiles and n items, fitted to measured times of
// forced split counts on this GPU (causal and not, B*H 1..32, N 512..32768; rms error 7.5%).  Items go to the slots
// in grid order, each to the slot that frees first (greedy list scheduling, as the dispatcher does).  An item costs
// 7.2 us (prologue, epilogue) plus, per key tile, max(0.76 us, r * 16 KiB / 6.7 TB/s) with r = min(n, slots) items
// running: the tile's compute, or every running item's K and V tile at the rate the caches and HBM sustain.  With
// s > 1 the merge adds 8.8 us plus the item's 128 rows of 1040-byte states read at 3.3 TB/s.
double split_plan_us(int64_t BH, int R, int K, int s, int kt, int causal, int64_t n) {
    const double tile_us = fmax(0.76, (double)(n < SPLIT_SLOTS ? n : SPLIT_SLOTS) * 16384.0 / 6.7e6);
    double slot[SPLIT_SLOTS] = {};   // min-heap of the slots' free times
    const auto later = [](double a, double b) { return a > b; };
    double end = 0.0;
    auto run = [&](int tiles, int64_t count) {
        const double cost = 7.2 + tiles * tile_us;
        for (int64_t c = 0; c < count; ++c) {
            std::pop_heap(slot, slot + SPLIT_SLOTS, later);
            slot[SPLIT_SLOTS - 1] += cost;
            end = fmax(end, slot[SPLIT_SLOTS - 1]);
            std::push_heap(slot, slot + SPLIT_SLOTS, later);
        }
    };
    int hi = R;
    for (int j = s; j >= 1; --j) {   // the kernel's item order (one group of all row tiles when not causal)
        const int lo = !causal ? 0 : j > 1 ? first_row_tile_with(j, kt, R) : 0;
        for (int rt = hi - 1; rt >= lo; --rt) {
            const int kend = !causal || rt == R - 1 ? K : (rt + 1) * (BM / BN);
            for (int64_t bh = 0; bh < BH; ++bh)
                for (int sp = 0; sp < j; ++sp) run(min(kend, (sp + 1) * kt) - sp * kt, 1);
        }
        hi = lo;
        if (!causal) break;
    }
    if (s > 1) end += 8.8 + (double)n * BM * 1040.0 / 3.3e6;
    return end;
}

int plan_key_splits(int64_t BH, int64_t N, int causal) {
    const int64_t rows = (N + BM - 1) / BM;
    const int R = (int)rows, K = (int)((N + BN - 1) / BN);
    int best = 1, last = 1;
    double best_t = split_plan_us(BH, R, K, 1, K, causal, rows * BH);
    for (int s0 = 2; s0 <= 16 && s0 <= K; ++s0) {
        const int kt = (K + s0 - 1) / s0, s = (K + kt - 1) / kt;   // as many splits as that share of key tiles needs
        if (s == last) continue;
        last = s;
        const int64_t n = split_items(BH, R, s, kt, causal);
        if (n > SPLIT_MAX_ITEMS) continue;
        const double t = split_plan_us(BH, R, K, s, kt, causal, n);
        if (t < best_t) {
            best_t = t;
            best = s;
        }
    }
    return best;
}

}  // namespace

// Key splits per row tile: the plan of least modelled time (split_plan_us) among 1..16 splits.  Launches whose row
// tiles alone fill the slots take 1.  The plan picked was within 15% of the fastest measured in every case measured
// (3.9% on average).  Plans are kept for the last few shapes, as the model takes up to a few hundred microseconds.
int prefill_key_splits(int64_t BH, int64_t N, int causal) {
    if (BH <= 0 || N <= 0 || BH * ((N + BM - 1) / BM) >= SPLIT_SLOTS) return 1;
    struct Plan {
        int64_t BH, N;
        int causal, splits;
    };
    static std::mutex mu;
    static Plan kept[16];
    static int kept_n = 0, next = 0;
    causal = causal ? 1 : 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < kept_n; ++i)
            if (kept[i].BH == BH && kept[i].N == N && kept[i].causal == causal) return kept[i].splits;
    }
    const int splits = plan_key_splits(BH, N, causal);
    std::lock_guard<std::mutex> lock(mu);
    kept[next] = Plan{BH, N, causal, splits};
    next = (next + 1) % 16;
    kept_n = kept_n < 16 ? kept_n + 1 : 16;
    return splits;
}

int prefill_key_splits_max(int64_t BH, int64_t N) {
    const int a = prefill_key_splits(BH, N, 0), b = prefill_key_splits(BH, N, 1);
    return a > b ? a : b;
}

hipError_t launch_prefill_split_bf16_d64(const uint16_t* q1, const uint16_t* k1, const uint16_t* q2,
                                         const uint16_t* k2, const uint16_t* v, uint16_t* out, int64_t B, int64_t H,
                                         int64_t N, int causal, Epilogue ep, float* part, hipStream_t stream) {
    const int64_t BH = B * H;
    const int splits = prefill_key_splits(BH, N, causal);
    const Strides st = contiguous_strides(H, N, D);
    if (splits <= 1) return launch_prefill_bf16_d64(q1, k1, q2, k2, v, out, B, H, N, causal, st, ep, nullptr, stream);
    const int n_row_tiles = (int)((N + BM - 1) / BM);
    const int key_tiles = (int)((N + BN - 1) / BN);
    const KeySplit ks{splits, (key_tiles + splits - 1) / splits, part};
    const int64_t blocks = split_items(BH, n_row_tiles, splits, ks.kt_split, causal);
    if (blocks > 0x7fffffff || BH * N > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_bf16_d64_kernel<false, true>), dim3((unsigned)blocks), dim3(THREADS), 0, stream, q1,
                       k1, q2, k2, v, out, (int)BH, (int)H, (int)N, n_row_tiles, causal ? 1 : 0, st, ep, nullptr, ks,
                       0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_merge_kernel, dim3((unsigned)((BH * N + 3) / 4)), dim3(256), 0, stream,
                       (const float*)part, out, (int)BH, (int)N, causal ? 1 : 0, splits, ks.kt_split, n_row_tiles, ep);
    return hipGetLastError();
}

}  // namespace diffattn
