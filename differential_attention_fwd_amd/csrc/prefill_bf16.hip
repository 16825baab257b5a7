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
//   * Loads go straight from global memory to LDS (buffer_load ... lds, no registers) through 4-slot rings: the
//     K1 and K2 tiles three tiles ahead, the raw V tile four ahead.  Every step transposes the next raw V tile
//     LDS-to-LDS (ds_read_b64_tr_b16, then 64-bit writes after the step's own work) into a channel-major V^T tile,
//     double-buffered, so that every MFMA operand is one 128-bit LDS read.  Ring slots are separate __shared__
//     arrays and the loop is unrolled by four, so the compiler can tell reads of one slot from loads still landing
//     in another.  One workgroup barrier per tile.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in
//     registers).  In the accumulator layout every lane owns ONE query row (lane % 32) and 16 of the 32 keys, so
//     row statistics need only the lane pair (l, l ^ 32), exchanged with v_permlane32_swap.
//   * P^T stays in registers and feeds O^T = V^T P^T directly as the MFMA B operand.  The k-order of that product
//     is the accumulator's key order; the transposed V tile stores keys in that order, so the A operand of each
//     MFMA is one contiguous 16-byte read, shared by the two maps.  O^T's layout gives each lane one query row
//     again, so the online-softmax rescale of O is lane-local.
//   * Two online softmaxes run side by side (running max and sum per map, two O accumulators).  The running max
//     only moves when a row's new maximum exceeds it by more than 2^8 (wave-uniform decision), so the O rescale
//     is rare; exponents use exp2 with log2(e)/sqrt(d) folded into one FMA; row sums add the bf16-rounded
//     probabilities pairwise with v_dot2_f32_bf16.  Map 2's exponentials are issued between map 1's value MFMAs.
//   * Epilogue: O1/l1 - lambda O2/l2, RMS over the 128 channels (pair-reduced), scale, bf16 round-to-nearest-even.
//   * Causal: row tiles are launched heaviest first; tiles wholly above a wave's rows are skipped by that wave,
//     and only diagonal or ragged-tail tiles pay for masking.
//
// This translation unit is compiled with -fno-honor-nans: no NaN can arise (inputs are finite, masked scores are
// -inf, and every processed row has a visible key in its first tile), and it lets v_max3 run without quieting.
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
constexpr int RING = 4;                         // ring slots: K tile t in slot t % 4 (loaded three tiles ahead),
                                                // raw V tile t in slot t % 4 (loaded four ahead)
constexpr int K_SLOT_BYTES = 2 * K_TILE_BYTES;

// Compile-time ring slot.  Each ring slot is its own __shared__ array, so the compiler can tell an LDS read of one
// slot from a direct load still landing in another and does not drain the prefetches before every LDS read.
template <int V> struct Slot { static constexpr int value = V; };
template <int S, class T> __device__ __forceinline__ T* pick4(T* a, T* b, T* c, T* d) {
    static_assert(RING == 4, "one array per ring slot");
    if constexpr (S % 4 == 0) return a;
    else if constexpr (S % 4 == 1) return b;
    else if constexpr (S % 4 == 2) return c;
    else return d;
}
constexpr float RESCALE_THRESHOLD = 8.0f;       // log2 units: p never exceeds 2^8 between rescales

__device__ __forceinline__ float max16(const f32x16& s) {
    const float a = fmaxf(fmaxf(s[0], s[1]), s[2]), b = fmaxf(fmaxf(s[3], s[4]), s[5]);
    const float c = fmaxf(fmaxf(s[6], s[7]), s[8]), d = fmaxf(fmaxf(s[9], s[10]), s[11]);
    const float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
    return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), s[15]));
}

// Online-softmax state of one map for the lane's query row.  The running max is kept in score units (ms) and in
// log2 units (ml = ms * c, the exponent offset); it only moves when a tile's max exceeds it by more than
// RESCALE_THRESHOLD log2 units (mt = ms + RESCALE_THRESHOLD / c), a wave-uniform decision, so the rescale of O and l
// is rare.
struct MapState {
    float ms, ml, mt, l;
};

__device__ __forceinline__ void update_max(const f32x16& s, MapState& st, f32x16 (&o)[4], float c, float thr) {
    const float x = pair_max(max16(s));
    if (__any(x > st.mt)) {
        const float ms = fmaxf(st.ms, x);
        const float ml = ms * c;
        const float alpha = __builtin_amdgcn_exp2f(st.ml - ml);
        st.ms = ms;
        st.ml = ml;
        st.mt = ms + thr;
        st.l *= alpha;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
    }
}

// p = exp2(s * c - ml) for the lane's 16 keys, packed as P^T: two bf16x8 B operands.
__device__ __forceinline__ void exp_pack(const f32x16& s, float ml, float c, bf16x8& lo, bf16x8& hi) {
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
}

// Adds the lane's 16 packed probabilities to l: pairwise bf16 dot products with (1, 1), so the sum is of the same
// bf16-rounded values that multiply V.
__device__ __forceinline__ float sum_packed(const bf16x8& lo, const bf16x8& hi, float l) {
    const u32x4 a = __builtin_bit_cast(u32x4, lo), b = __builtin_bit_cast(u32x4, hi);
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const unsigned ak = a[k], bk = b[k];   // scalar copies: bit_cast of a vector element misreads it
        t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ak), one, t0, false);
        t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, bk), one, t1, false);
    }
    return l + (t0 + t1);
}

// SAVE: also write each row's training statistics (SAVED_* in launch.h) for the backward pass.
template <bool SAVE>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_d64_kernel(const uint16_t* __restrict__ gq1, const uint16_t* __restrict__ gk1,
                             const uint16_t* __restrict__ gq2, const uint16_t* __restrict__ gk2,
                             const uint16_t* __restrict__ gv, uint16_t* __restrict__ gout, int BH, int H, int N,
                             int n_row_tiles, int causal, Strides st, Epilogue ep, float* __restrict__ saved) {
    __shared__ __attribute__((aligned(16))) unsigned char kr0[K_SLOT_BYTES], kr1[K_SLOT_BYTES], kr2[K_SLOT_BYTES],
        kr3[K_SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char vr0[V_TILE_BYTES], vr1[V_TILE_BYTES], vr2[V_TILE_BYTES],
        vr3[V_TILE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char vtb[2 * V_TILE_BYTES];   // transposed V, double buffer

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int h = lane >> 5;     // which half of the accumulator's key rows this lane holds
    const int l32 = lane & 31;   // this lane's query row inside the wave

    // Heaviest row tiles first under the causal mask (their key range is longest).
    const int bid = blockIdx.x;
    const int rt = causal ? (n_row_tiles - 1 - bid / BH) : bid / BH;
    const int bh = bid % BH;
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

    // Direct loads: each wave moves one 1 KiB piece per tile and tensor role.  K1 and K2 tiles (4 KiB each) are 8
    // pieces, the raw V tile (8 KiB) another 8; piece x of a tile covers its bytes [1024 x, 1024 x + 1024) and lane L
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
        // K tile row 8 (piece % 4) + L / 8, stored chunk L % 8 = logical chunk ^ ((row >> 1) & 7) (see k_off).
        const int row = 8 * (piece & 3) + (lane >> 3);
        kd_voff[j] = (unsigned)row * rb + ((((lane & 7) ^ ((row >> 1) & 7))) << 4);
        kd_step[j] = (unsigned)BN * rb;            // bytes per tile
        kd_lds[j] = (piece >> 2) * K_TILE_BYTES + 1024 * (piece & 3);
    }
#pragma unroll
    for (int j = 0; j < V_PIECES_PER_WAVE; ++j) {
        // Raw V: position p holds row p / 256 and stored chunk (p / 16) % 16 = logical chunk ^ (2 (row & 3)).
        const int p = 1024 * (wave + WAVES * j) + 16 * lane;
        const int row = p >> 8, pchunk = (p >> 4) & 15;
        vd_voff[j] = (unsigned)row * vrb + ((pchunk ^ ((row & 3) << 1)) << 4);
    }
    const unsigned vd_step = (unsigned)BN * vrb;
    // Transpose raw V -> V^T with ds_read_b64_tr_b16.  A 16-lane group reads a block of 4 keys x 16 channels (lane
    // 4 jj + q supplies key jj, channels 4 q .. 4 q + 3) and lane i receives channel i of the block for the 4 keys:
    // 8 bytes of one V^T row, stored with one 64-bit write.  The 64 blocks of a tile are shared out over the
    // workgroup's 16-lane groups: group g takes blocks g + GROUPS b (keys 4 ((g + GROUPS b) / 8) .. + 3, channels
    // 16 (g % 8) .. + 15); consecutive blocks of a group lie (GROUPS / 8) x 1 KiB apart in the raw tile.
    constexpr int GROUPS = THREADS / 16;
    constexpr int TR_BLOCKS = 64 / GROUPS;
    const int grp = tid >> 4, gl = tid & 15;
    const int cgb = grp & 7;
    const int tr_ch = 16 * cgb + 4 * (gl & 3);   // first channel of the 8 bytes this lane supplies
    const int tr_rd = vr_off(4 * (grp >> 3) + (gl >> 2), tr_ch >> 3) + (tr_ch & 7) * 2;
    int tr_wr[TR_BLOCKS];
#pragma unroll
    for (int b = 0; b < TR_BLOCKS; ++b) {
        const int pos = key_pos(4 * ((grp + GROUPS * b) >> 3));   // the block's 4 keys sit at 4 consecutive positions
        tr_wr[b] = vt_off(16 * cgb + gl, pos >> 3) + (pos & 7) * 2;
    }

    auto vslot = [&](int t) { return vtb + (t & 1) * V_TILE_BYTES; };
    auto issue_k = [&](auto S, int t) {   // S = t % 4
        unsigned char* slot = pick4<decltype(S)::value>(kr0, kr1, kr2, kr3);
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
        for (int j = 0; j < V_PIECES_PER_WAVE; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(slot + 1024 * (wave + WAVES * j)), 16,
                                                     (int)(vd_voff[j] + (unsigned)t * vd_step), 0, 0, 0);
    };
    // Transposition of raw V slot S into the V^T buffer of tile t, in two steps (read, then write) so that the
    // tile's computation hides the latency of the transposing reads.
    s16x4 trx[TR_BLOCKS];
    auto transpose_read = [&](auto S) {
        const unsigned char* raw = pick4<decltype(S)::value>(vr0, vr1, vr2, vr3);
#pragma unroll
        for (int b = 0; b < TR_BLOCKS; ++b)
            trx[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(raw + tr_rd + (GROUPS / 8) * 1024 * b));
    };
    auto transpose_write = [&](int t) {
        unsigned char* vt = vslot(t);
#pragma unroll
        for (int b = 0; b < TR_BLOCKS; ++b) *(s16x4*)(vt + tr_wr[b]) = trx[b];
    };

    // Per-lane read offsets: K A-operand (row l32, chunk 2 kc + h) and V^T A-operand (channel 32 cb + l32,
    // chunk 2 ks + h; the four channel blocks are 2 KiB apart).
    // k_off(l32, 2 kc + h) = k_rd0 ^ (32 kc): the chunk swizzle is an XOR on bits 4..6 of the offset.
    const int k_rd0 = k_off(l32, h);
    const int v_rd0 = vt_off(l32, h);
    const int v_rd1 = vt_off(l32, 2 + h);

    f32x16 o1[4], o2[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) { o1[cb][i] = 0.f; o2[cb][i] = 0.f; }
    const float c = LOG2E * 0.125f;  // log2(e) / sqrt(64)
    const float thr = RESCALE_THRESHOLD / c;
    MapState st1 = {-INFINITY, -INFINITY, -INFINITY, 0.f}, st2 = st1;

    // Load schedule.  Iteration t (between two workgroup barriers) issues the direct loads of K(t + 2) and raw
    // V(t + 3), transposes raw V(t + 1) into the V^T buffer of tile t + 1, and computes tile t.  At its end it waits
    // for everything but its own loads, so a load issued in iteration u is usable from iteration u + 1 on
    // (and has had the whole of iteration u to land).
    issue_k(Slot<0>{}, 0);
    issue_v(Slot<0>{}, 0);
    issue_k(Slot<1>{}, 1);
    issue_v(Slot<1>{}, 1);
    issue_k(Slot<2>{}, 2);
    issue_v(Slot<2>{}, 2);
    issue_v(Slot<3>{}, 3);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    lds_barrier();
    transpose_read(Slot<0>{});
    transpose_write(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    lds_barrier();
    auto step = [&](auto S, int t) {   // S = t % 4
        constexpr int s0 = decltype(S)::value;
        issue_k(Slot<(s0 + 3) % 4>{}, t + 3);
        issue_v(Slot<s0>{}, t + 4);
        transpose_read(Slot<(s0 + 1) % 4>{});
        const int kv0 = t * BN;
        if (!causal || kv0 <= q0w + 31) {
            const unsigned char* kb_ = pick4<s0>(kr0, kr1, kr2, kr3);
            const unsigned char* vb_ = vslot(t);
            f32x16 s1, s2;
#pragma unroll
            for (int i = 0; i < 16; ++i) { s1[i] = 0.f; s2[i] = 0.f; }
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const int kro = k_rd0 ^ (32 * kc);
                const bf16x8 ka = *(const bf16x8*)(kb_ + kro);
                const bf16x8 kb = *(const bf16x8*)(kb_ + K_TILE_BYTES + kro);
                s1 = mfma(ka, qa[kc], s1);
                s2 = mfma(kb, qb[kc], s2);
            }
            if ((causal && kv0 + BN - 1 > q0w) || kv0 + BN > N) {
                const int q = q0w + l32;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kv0 + 8 * (i >> 2) + 4 * h + (i & 3);
                    const bool vis = key < N && (!causal || key <= q);
                    s1[i] = vis ? s1[i] : -INFINITY;
                    s2[i] = vis ? s2[i] : -INFINITY;
                }
            }
            update_max(s1, st1, o1, c, thr);
            update_max(s2, st2, o2, c, thr);

            bf16x8 p1[2], p2[2];
            exp_pack(s1, st1.ml, c, p1[0], p1[1]);
            bf16x8 va[4][2];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) va[cb][0] = *(const bf16x8*)(vb_ + v_rd0 + 2048 * cb);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o1[cb] = mfma(va[cb][0], p1[0], o1[cb]);
            exp_pack(s2, st2.ml, c, p2[0], p2[1]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) va[cb][1] = *(const bf16x8*)(vb_ + v_rd1 + 2048 * cb);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o2[cb] = mfma(va[cb][0], p2[0], o2[cb]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o1[cb] = mfma(va[cb][1], p1[1], o1[cb]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o2[cb] = mfma(va[cb][1], p2[1], o2[cb]);
            st1.l = sum_packed(p1[0], p1[1], st1.l);
            st2.l = sum_packed(p2[0], p2[1], st2.l);
        }
        transpose_write(t + 1);
        // The loads of this iteration and the previous one (K(t + 2), V(t + 3), K(t + 3), V(t + 4)) may stay in
        // flight past the barrier; everything older, in particular K(t + 1) and V(t + 2), has landed, and the
        // transposed V(t + 1) is written.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * (K_PIECES_PER_WAVE + V_PIECES_PER_WAVE)));
        lds_barrier();
    };
    for (int t = 0; t < n_tiles; t += 4) {
        step(Slot<0>{}, t);
        if (t + 1 < n_tiles) step(Slot<1>{}, t + 1);
        if (t + 2 < n_tiles) step(Slot<2>{}, t + 2);
        if (t + 3 < n_tiles) step(Slot<3>{}, t + 3);
    }
    // Drain the trailing prefetches before the workgroup can retire (their LDS writes must not outlive it).
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

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

}  // namespace

hipError_t launch_prefill_bf16_d64(const uint16_t* q1, const uint16_t* k1, const uint16_t* q2, const uint16_t* k2,
                                   const uint16_t* v, uint16_t* out, int64_t B, int64_t H, int64_t N, int causal,
                                   const Strides& st, Epilogue ep, float* saved, hipStream_t stream) {
    const int64_t BH = B * H;
    const int n_row_tiles = (int)((N + BM - 1) / BM);
    const int64_t blocks = (int64_t)n_row_tiles * BH;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (saved)
        hipLaunchKernelGGL(prefill_bf16_d64_kernel<true>, dim3((unsigned)blocks), dim3(THREADS), 0, stream, q1, k1,
                           q2, k2, v, out, (int)BH, (int)H, (int)N, n_row_tiles, causal ? 1 : 0, st, ep, saved);
    else
        hipLaunchKernelGGL(prefill_bf16_d64_kernel<false>, dim3((unsigned)blocks), dim3(THREADS), 0, stream, q1, k1,
                           q2, k2, v, out, (int)BH, (int)H, (int)N, n_row_tiles, causal ? 1 : 0, st, ep, saved);
    return hipGetLastError();
}

}  // namespace diffattn
