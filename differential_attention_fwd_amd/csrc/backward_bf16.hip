// Backward pass of differential attention for gfx950 (bf16 inputs and gradients, fp32 accumulation, d = 64,
// 2d = 128).
//
// The forward it differentiates (Ultralytics glossary "Differential Transformer", section on how differential
// attention works: worked example and the paragraph after it): per head and query row i, a = softmax(q1 K1^T /
// sqrt(d)), b = softmax(q2 K2^T / sqrt(d)), o = (a - lambda b) V, then for layer >= 1 the RMS normalisation and
// the (1 - lambda_init) scale.  The pages give no backward pass; these kernels apply the chain rule:
//   dO  = g r dy - g r^3 o (dy . o) / 2d        (normalised layers; g = 1 - lambda_init, r = (mean o^2 + eps)^-1/2)
//   E1  = dO . o1,  E2 = dO . o2                 (o1 = a V, o2 = b V, saved by the training forward)
//   dp  = dO . v_j
//   ds1 = a (dp - E1),   ds2 = -lambda b (dp - E2)
//   dV  = sum_i (a - lambda b)_ij dO_i,   dQ1 = ds1 K1 / sqrt(d),   dK1 = ds1^T Q1 / sqrt(d)   (same for map 2)
//   dlambda = -sum_i dO_i . o2_i                  (per head, summed over the batch)
// with a and b recomputed from the scores and the per-row log-sum-exps saved by the forward.
//
// Kernels (all launched on one stream, in order):
//   1. bwd_pre:      per row, dO (bf16) and (lse1, lse2, E1, E2), and the row's share of dlambda.
//   2. bwd_dq:       per 128-row query block (4 waves x 32 rows), loop over key tiles up to the diagonal:
//                    S^T = K Q^T and dP^T = V dO^T on MFMA, ds in registers, dQ^T += K^T ds^T with the K^T
//                    operands read from the row-major K tiles with ds_read_b64_tr_b16.  Same register plan and
//                    load rings as the forward (two waves per SIMD).
//   3. bwd_dkdv:     per 64-key block (4 waves x 16 keys, v_mfma_f32_16x16x32_bf16), loop over query tiles from the
//                    diagonal: S = Q K^T and dP = dO V^T with the wave's K and V rows held in registers, then
//                    dV^T += dO^T W and dK^T += Q^T ds, the transposed operands read from the row-major tiles with
//                    ds_read_b64_tr_b16.  Three waves per SIMD.  Q, dO and stats tiles come straight from global
//                    memory to LDS (buffer_load ... lds) through a 3-slot ring, two tiles ahead, one barrier per
//                    tile.
//   4. bwd_dlambda:  per head, a fixed-order sum of the rows' dlambda shares (deterministic).

#include "launch.h"
#include "tiles.h"

namespace diffattn {
namespace {

constexpr int D = 64;
constexpr int DV = 128;
constexpr int TILE = 32;          // keys (dq) or queries (dkdv) per tile
constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int BLOCK = TILE * WAVES;   // rows (dq) or keys (dkdv) per workgroup
constexpr int STAT_FLOATS = 4;    // per row in the workspace: lse1, lse2, E1, E2

// ---------------------------------------------------------------------------------------------------------------
// LDS tile layouts and helpers shared by the dQ and dK/dV kernels.
// ---------------------------------------------------------------------------------------------------------------
// The LDS has 64 banks of 4 bytes.  A 64-bit read (the transposing ones included) is served in two windows of 32
// consecutive lanes; a 128-bit read in four windows of 16 lanes: within each half wave, the 4-lane groups
// q = (lane >> 2) & 7 of even bit parity form one window and those of odd parity the other (measured on gfx950
// with pairs of active lanes).  A read takes one pass per window when the window's lanes touch distinct banks.
//
// Q tile (and the dQ kernel's K tiles): row r of 128 bytes; chunk c at c ^ q_sw(r), q_sw linear over GF(2) in
// x = (r >> 1) & 7.  Found by exhaustive search over such maps: free of conflicts for the 16-row 128-bit reads (dK/dV:
// 16 rows x 4 chunks; dQ: 32 rows x 2 chunks) and the 32-lane transposing reads (dK/dV: 8 rows x 2 adjacent chunks;
// dQ: 4 rows x 4 chunks).
__device__ __forceinline__ int q_sw(int r) {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) ^ (((x >> 1) & 1) * 3) ^ (((x >> 2) & 1) << 1);
}
__device__ __forceinline__ int q_off(int r, int c) { return r * 128 + ((c ^ q_sw(r)) << 4); }
// dO tile (and the dQ kernel's V tiles): row r of 256 bytes; chunk c at c ^ do_sw(r), linear in the bits of r % 16,
// found the same way for the 16-row 128-bit reads (dK/dV: 16 rows x 4 chunks; dQ: 32 rows x 2 chunks) and the
// 32-lane transposing reads of 8 rows x 2 adjacent chunks.
__device__ __forceinline__ int do_sw(int r) {
    return ((r & 1) << 3) ^ (((r >> 1) & 1) << 2) ^ (((r >> 2) & 1) * 3) ^ (((r >> 3) & 1) << 1);
}
__device__ __forceinline__ int do_off(int r, int c) { return r * 256 + ((c ^ do_sw(r)) << 4); }

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int V> struct Slot { static constexpr int value = V; };
template <int S, class T> __device__ __forceinline__ T* pick3(T* a, T* b, T* c) {
    if constexpr (S % 3 == 0) return a;
    else if constexpr (S % 3 == 1) return b;
    else return c;
}
template <int S, class T> __device__ __forceinline__ T* pick4(T* a, T* b, T* c, T* d) {
    if constexpr (S % 4 == 0) return a;
    else if constexpr (S % 4 == 1) return b;
    else if constexpr (S % 4 == 2) return c;
    else return d;
}

__device__ __forceinline__ unsigned pack_bf16_bits(float a, float b) { return pack2(a, b); }

// ---------------------------------------------------------------------------------------------------------------
// 1. Preprocess: 16 lanes per row (4 rows per wave); lane q of a row holds channels 8 q .. 8 q + 7, so every load and
//    store is 16 bytes wide and each dot product needs a 4-step reduction over the row's 16 lanes.
// ---------------------------------------------------------------------------------------------------------------
constexpr int PRE_ROWS = 4 * WAVES;   // rows per workgroup

__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m, 16);
    return x;
}

__global__ __launch_bounds__(THREADS) void bwd_pre_kernel(const uint16_t* __restrict__ dy, const float* __restrict__ saved,
                                                          uint16_t* __restrict__ dO, float* __restrict__ stats,
                                                          float* __restrict__ dl_rows, int64_t rows, int N, int H,
                                                          BwdStrides gs, Epilogue ep) {
    const int q = threadIdx.x & 15;
    const int64_t row_u = (int64_t)blockIdx.x * PRE_ROWS + (threadIdx.x >> 4);
    const bool live = row_u < rows;
    const int64_t row = live ? row_u : rows - 1;   // tail lanes redo the last row and store nothing
    const int bh = (int)(row / N);
    const float lam = lambda_of(ep, bh);
    const float* srow = saved + row * SAVED_FLOATS;
    const int64_t i = row - (int64_t)bh * N;
    const u32x4 dyw = *(const u32x4*)(dy + (bh / H) * gs.b[G_DY] + (bh % H) * gs.h[G_DY] + i * gs.n[G_DY] + 8 * q);
    const f32x4 o1a = *(const f32x4*)(srow + SAVED_O1 + 8 * q), o1b = *(const f32x4*)(srow + SAVED_O1 + 8 * q + 4);
    const f32x4 o2a = *(const f32x4*)(srow + SAVED_O2 + 8 * q), o2b = *(const f32x4*)(srow + SAVED_O2 + 8 * q + 4);
    const f32x4 hdr = *(const f32x4*)srow;   // lse1, lse2, r, unused
    float y[8], o1[8], o2[8], oc[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const unsigned w = dyw[k];
        y[2 * k] = __uint_as_float(w << 16);
        y[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
        o1[k] = o1a[k];
        o1[4 + k] = o1b[k];
        o2[k] = o2a[k];
        o2[4 + k] = o2b[k];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) oc[c] = o1[c] - lam * o2[c];
    float d[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) d[c] = y[c];
    if (ep.normalise) {
        const float rr = hdr[2];
        float t = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) t += y[c] * oc[c];
        const float dyo = row16_sum(t);
        const float g = ep.out_scale;
        const float k = g * rr * rr * rr * dyo * (1.f / DV);
#pragma unroll
        for (int c = 0; c < 8; ++c) d[c] = g * rr * y[c] - k * oc[c];
    }
    // dO is used in bf16 by the matrix products; E1 and E2 use the same rounded values.
    u32x4 db;
#pragma unroll
    for (int k = 0; k < 4; ++k) db[k] = pack_bf16_bits(d[2 * k], d[2 * k + 1]);
    if (live) *(u32x4*)(dO + row * DV + 8 * q) = db;
    float e1 = 0.f, e2 = 0.f, dl = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const unsigned w = db[k];
        const float r0 = __uint_as_float(w << 16), r1 = __uint_as_float(w & 0xffff0000u);
        e1 += r0 * o1[2 * k] + r1 * o1[2 * k + 1];
        e2 += r0 * o2[2 * k] + r1 * o2[2 * k + 1];
    }
    // dlambda is a sum over rows with much cancellation: it uses the unrounded dO.
#pragma unroll
    for (int c = 0; c < 8; ++c) dl += d[c] * o2[c];
    e1 = row16_sum(e1);
    e2 = row16_sum(e2);
    dl = row16_sum(dl);
    if (live && q == 0) {
        *(f32x4*)(stats + row * STAT_FLOATS) = f32x4{hdr[0], hdr[1], e1, e2};
        dl_rows[row] = -dl;
    }
}

// ---------------------------------------------------------------------------------------------------------------
// 2. dQ: per 128-row query block; lane owns query row q0w + l32 (as in the forward).
// ---------------------------------------------------------------------------------------------------------------
// K1, K2 and V tiles come straight from global memory to LDS (buffer_load ... lds) through 4-slot rings, three
// tiles ahead, one barrier per tile.  K tiles use the q_sw swizzle (16-row 128-bit reads for S^T = K Q^T and
// 4-row transposing reads for dQ^T += K^T ds^T are both free of bank conflicts); the V tile, read only by rows for
// dP^T = V dO^T, uses do_sw.
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const uint16_t* __restrict__ gq1, const uint16_t* __restrict__ gk1,
                   const uint16_t* __restrict__ gq2, const uint16_t* __restrict__ gk2,
                   const uint16_t* __restrict__ gv, const uint16_t* __restrict__ gdo,
                   const float* __restrict__ stats, uint16_t* __restrict__ dq1, uint16_t* __restrict__ dq2,
                   int BH, int N, int n_blocks, int causal, int H, BwdStrides gs, Epilogue ep, int xcd_group) {
    constexpr int K_TILE = TILE * D * 2, V_TILE = TILE * DV * 2;
    __shared__ __attribute__((aligned(16))) unsigned char kr0[2 * K_TILE], kr1[2 * K_TILE], kr2[2 * K_TILE],
        kr3[2 * K_TILE];
    __shared__ __attribute__((aligned(16))) unsigned char vr0[V_TILE], vr1[V_TILE], vr2[V_TILE], vr3[V_TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    int r, bh;   // heaviest query blocks first; each XCD's heads a group at a time (xcd_item)
    xcd_item((int)blockIdx.x, BH, n_blocks, xcd_group, r, bh);
    const int qb = causal ? (n_blocks - 1 - r) : r;
    const int q0 = qb * BLOCK, q0w = q0 + TILE * wave;
    const size_t hv = (size_t)bh * N * DV;   // the workspace's dO rows
    const int64_t b_ = bh / H, h_ = bh % H;
    auto gbase = [&](int k) { return b_ * gs.b[k] + h_ * gs.h[k]; };   // head's first element of caller tensor k
    const int q = q0w + l32, qc = min(q, N - 1);
    const float c = LOG2E * 0.125f;

    // Per-head buffer resources over the head's rows (row strides in bytes): rows at or beyond N read as zero.  The
    // caller checked that N + 256 rows fit the unsigned 32-bit offsets.
    const unsigned rbk1 = (unsigned)gs.n[G_K1] * 2u, rbk2 = (unsigned)gs.n[G_K2] * 2u, rbv = (unsigned)gs.n[G_V] * 2u;
    const unsigned n1 = (unsigned)(N - 1);
    const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc((void*)(gk1 + gbase(G_K1)), (short)0,
                                                                         (int)(n1 * rbk1 + D * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rk2 = __builtin_amdgcn_make_buffer_rsrc((void*)(gk2 + gbase(G_K2)), (short)0,
                                                                         (int)(n1 * rbk2 + D * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(gv + gbase(G_V)), (short)0,
                                                                        (int)(n1 * rbv + DV * 2u), 0x00020000);

    // Direct loads per wave and tile: K1 rows 8 wave .. + 7, K2 the same, V rows 4 p .. 4 p + 3 for pieces
    // p = wave and wave + 4 (lane L writes position 16 L of a 1 KiB piece).  Issued unconditionally, also past the
    // end (out of range: zeros), so every iteration issues the same number.
    const int krow = 8 * wave + (lane >> 3);
    const unsigned k_chunk = (((lane & 7) ^ q_sw(krow))) << 4;
    const unsigned k1_voff = (unsigned)krow * rbk1 + k_chunk, k2_voff = (unsigned)krow * rbk2 + k_chunk;
    const unsigned k1_step = TILE * rbk1, k2_step = TILE * rbk2, v_step = TILE * rbv;   // bytes per tile
    unsigned v_voff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 4 * (wave + WAVES * j) + (lane >> 4);
        v_voff[j] = (unsigned)r * rbv + ((((lane & 15) ^ do_sw(r))) << 4);
    }
    auto issue = [&](auto S, int t) __attribute__((always_inline)) {
        constexpr int s0 = decltype(S)::value;
        unsigned char* ks = pick4<s0>(kr0, kr1, kr2, kr3);
        unsigned char* vs = pick4<s0>(vr0, vr1, vr2, vr3);
        check_fill(ks + 1024 * wave, 16);
        check_fill(ks + K_TILE + 1024 * wave, 16);
#pragma unroll
        for (int j = 0; j < 2; ++j) check_fill(vs + 1024 * (wave + WAVES * j), 16);
        check_fence();
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk1, (lds_void*)(ks + 1024 * wave), 16,
                                                 (int)(k1_voff + (unsigned)t * k1_step), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk2, (lds_void*)(ks + K_TILE + 1024 * wave), 16,
                                                 (int)(k2_voff + (unsigned)t * k2_step), 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vs + 1024 * (wave + WAVES * j)), 16,
                                                     (int)(v_voff[j] + (unsigned)t * v_step), 0, 0, 0);
    };
    constexpr int DQ_LOADS = 4;

    const int q_last = min(N, q0 + BLOCK) - 1;
    const int n_tiles = causal ? (q_last / TILE + 1) : (N + TILE - 1) / TILE;
    const int t_last = causal ? min(n_tiles - 1, (q0w + TILE - 1) / TILE) : n_tiles - 1;
    issue(Slot<0>{}, 0);
    issue(Slot<1>{}, 1);
    issue(Slot<2>{}, 2);

    // The wave's Q1, Q2 and dO rows as B operands and the row's statistics; loaded after the first tiles' direct
    // loads and used before the loop, so the compiler places no wait for them inside it.
    bf16x8 qa[4], qbf[4], dob[8];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        qa[kc] = *(const bf16x8*)(gq1 + gbase(G_Q1) + qc * gs.n[G_Q1] + 16 * kc + 8 * h);
        qbf[kc] = *(const bf16x8*)(gq2 + gbase(G_Q2) + qc * gs.n[G_Q2] + 16 * kc + 8 * h);
    }
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) dob[kc] = *(const bf16x8*)(gdo + hv + (size_t)qc * DV + 16 * kc + 8 * h);
    f32x4 st = *(const f32x4*)(stats + ((size_t)bh * N + qc) * STAT_FLOATS);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) asm volatile("" ::"v"(qa[kc]), "v"(qbf[kc]));
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) asm volatile("" ::"v"(dob[kc]));
    asm volatile("" ::"v"(st));
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    const float lse1 = st[0], lse2 = st[1], e1 = st[2], e2 = st[3];

    f32x16 acc1[2], acc2[2];   // dQ^T blocks: d = 32 mb + 8 (i / 4) + 4 h + i % 4, query = lane's row
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) { acc1[mb][i] = 0.f; acc2[mb][i] = 0.f; }

    // Read offsets.  S^T's A operand: K row l32, chunk 2 kc + h: q_off(l32, 2 kc + h) = k_rd0 ^ (32 kc).  dP^T's
    // A operand: V row l32, chunk 2 kc + h: do_off(l32, 2 kc + h) = v_rd0 ^ (32 kc).  dQ^T's A operand (K^T, feature
    // block mb, key half ks): lane 4 jj + qq of 16-lane group G supplies key row 16 ks + 4 h + jj (first read) or
    // 16 ks + 8 + 4 h + jj (second), features 32 mb + 16 (G & 1) + 4 qq .. + 3, and receives feature
    // 32 mb + l32 of those 4 keys; mb XORs 64 mb into the offset, ks adds 2 KiB.
    const int k_rd0 = q_off(l32, h), v_rd0 = do_off(l32, h);
    const int grp = (lane >> 4) & 1, jj = (lane >> 2) & 3, qq = lane & 3;
    const int kt_a = q_off(4 * h + jj, 2 * grp + (qq >> 1)) + 8 * (qq & 1);
    const int kt_b = q_off(8 + 4 * h + jj, 2 * grp + (qq >> 1)) + 8 * (qq & 1);
    auto kt_frag = [&](const unsigned char* p, int mb, int ks) __attribute__((always_inline)) {
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + (kt_a ^ (64 * mb)) + 2048 * ks));
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + (kt_b ^ (64 * mb)) + 2048 * ks));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    auto step = [&](auto S, int t) __attribute__((always_inline)) {   // S = t % 4
        constexpr int s0 = decltype(S)::value;
        issue(Slot<(s0 + 3) % 4>{}, t + 3);
        if (t <= t_last) {
            const unsigned char* k1s = pick4<s0>(kr0, kr1, kr2, kr3);
            const unsigned char* k2s = k1s + K_TILE;
            const unsigned char* vs = pick4<s0>(vr0, vr1, vr2, vr3);
            __builtin_amdgcn_s_setprio(1);
            // S^T = K Q^T (both maps) and dP^T = V dO^T: lane holds query q, keys t*32 + 8 (i/4) + 4 h + i % 4.
            f32x16 s1, s2, dp;
#pragma unroll
            for (int i = 0; i < 16; ++i) { s1[i] = 0.f; s2[i] = 0.f; dp[i] = 0.f; }
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                s1 = mfma(*(const bf16x8*)(k1s + (k_rd0 ^ (32 * kc))), qa[kc], s1);
                s2 = mfma(*(const bf16x8*)(k2s + (k_rd0 ^ (32 * kc))), qbf[kc], s2);
            }
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) dp = mfma(*(const bf16x8*)(vs + (v_rd0 ^ (32 * kc))), dob[kc], dp);
            __builtin_amdgcn_s_setprio(0);
            const int kv0 = t * TILE;
            const bool edge = (causal && kv0 + TILE - 1 > q0w) || kv0 + TILE > N;
            float g1[16], g2[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -lse1));
                const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[i], c, -lse2));
                g1[i] = a * (dp[i] - e1);
                g2[i] = b * (dp[i] - e2);   // times -lambda at the end
            }
            if (edge) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kv0 + 8 * (i >> 2) + 4 * h + (i & 3);
                    const bool vis = key < N && (!causal || key <= q);
                    g1[i] = vis ? g1[i] : 0.f;
                    g2[i] = vis ? g2[i] : 0.f;
                }
            }
            bf16x8 p1[2], p2[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u32x4 a, b;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    a[k] = pack2(g1[8 * ks + 2 * k], g1[8 * ks + 2 * k + 1]);
                    b[k] = pack2(g2[8 * ks + 2 * k], g2[8 * ks + 2 * k + 1]);
                }
                p1[ks] = __builtin_bit_cast(bf16x8, a);
                p2[ks] = __builtin_bit_cast(bf16x8, b);
            }
            __builtin_amdgcn_s_setprio(1);
            // dQ^T += K^T ds^T.
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    acc1[mb] = mfma(kt_frag(k1s, mb, ks), p1[ks], acc1[mb]);
                    acc2[mb] = mfma(kt_frag(k2s, mb, ks), p2[ks], acc2[mb]);
                }
            __builtin_amdgcn_s_setprio(0);
        }
        // The loads of this iteration and the previous one may stay in flight past the barrier; tile t + 1 has
        // landed.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * DQ_LOADS));
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
    if (q >= N) return;
    const float sc1 = 0.125f, sc2 = -lambda_of(ep, bh) * 0.125f;
    uint16_t* r1 = dq1 + gbase(G_DQ1) + q * gs.n[G_DQ1] + 4 * h;
    uint16_t* r2 = dq2 + gbase(G_DQ2) + q * gs.n[G_DQ2] + 4 * h;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            u32x2 w1, w2;
            w1[0] = pack2(acc1[mb][4 * g4] * sc1, acc1[mb][4 * g4 + 1] * sc1);
            w1[1] = pack2(acc1[mb][4 * g4 + 2] * sc1, acc1[mb][4 * g4 + 3] * sc1);
            w2[0] = pack2(acc2[mb][4 * g4] * sc2, acc2[mb][4 * g4 + 1] * sc2);
            w2[1] = pack2(acc2[mb][4 * g4 + 2] * sc2, acc2[mb][4 * g4 + 3] * sc2);
            *(u32x2*)(r1 + 32 * mb + 8 * g4) = w1;
            *(u32x2*)(r2 + 32 * mb + 8 * g4) = w2;
        }
}

// ---------------------------------------------------------------------------------------------------------------
// 3. dK, dV: per 64-key block (4 waves x 16 keys); lane owns key k0w + (lane % 16) in every product.
// ---------------------------------------------------------------------------------------------------------------
// Products per 32-query tile, all with v_mfma_f32_16x16x32_bf16 (A 16 x 32: lane holds A[m = l % 16][k = 8 (l / 16)
// + j]; B 32 x 16: lane holds B[k = 8 (l / 16) + j][n = l % 16]; D 16 x 16: lane holds D[m = 4 (l / 16) + i][n = l %
// 16]), in 16-query blocks mb:
//   S = Q K^T and dP = dO V^T: A = Q or dO rows from LDS, B = the wave's K^T or V^T held in registers.  Lane l then
//   holds key l % 16 and queries 16 mb + 4 g + i (g = l / 16), so a lane's 8 values of W = a - lambda b, ds1 and
//   ds2 over the two blocks are, in order, exactly the B operand (k = queries 4 g + 0..3, then 16 + 4 g + 0..3)
//   of the next products:
//   dV^T += dO^T W and dK^T += Q^T ds: A = dO^T or Q^T (one feature, those 8 queries per lane) from two
//   ds_read_b64_tr_b16 reads of the row-major tile.
// The Q and dO tiles are swizzled so that both the 16-row 128-bit reads and the 4-row transposing reads hit
// distinct LDS bank quads.
constexpr int KW = 16;                            // keys per wave
constexpr int KBLK = KW * WAVES;                  // keys per workgroup
constexpr int Q_TILE_BYTES = TILE * D * 2;        // 4 KiB
constexpr int DO_TILE_BYTES = TILE * DV * 2;      // 8 KiB
constexpr int ST_TILE_BYTES = TILE * STAT_FLOATS * 4;
constexpr int SLOT_BYTES = 2 * Q_TILE_BYTES + DO_TILE_BYTES + ST_TILE_BYTES;   // Q1 | Q2 | dO | stats
constexpr int ST_OFF = 2 * Q_TILE_BYTES + DO_TILE_BYTES;
constexpr int DKDV_LOADS = 5;                     // direct loads per wave and tile: Q1, Q2, 2 x dO, stats

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(3, 3)))
void bwd_dkdv_kernel(const uint16_t* __restrict__ gq1, const uint16_t* __restrict__ gk1,
                     const uint16_t* __restrict__ gq2, const uint16_t* __restrict__ gk2,
                     const uint16_t* __restrict__ gv, const uint16_t* __restrict__ gdo,
                     const float* __restrict__ stats, uint16_t* __restrict__ dk1, uint16_t* __restrict__ dk2,
                     uint16_t* __restrict__ dv, int BH, int N, int causal, int H, BwdStrides gs, Epilogue ep,
                     int xcd_group) {
    __shared__ __attribute__((aligned(16))) unsigned char sl0[SLOT_BYTES], sl1[SLOT_BYTES], sl2[SLOT_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // Key blocks in order (the first ones see the most queries under the causal mask); each XCD's heads a group at
    // a time (xcd_item).
    int kb, bh;
    xcd_item((int)blockIdx.x, BH, (N + KBLK - 1) / KBLK, xcd_group, kb, bh);
    const int k0 = kb * KBLK, k0w = k0 + KW * wave;
    const size_t hv = (size_t)bh * N * DV;   // the workspace's dO rows
    const int64_t b_ = bh / H, h_ = bh % H;
    auto gbase = [&](int k) { return b_ * gs.b[k] + h_ * gs.h[k]; };   // head's first element of caller tensor k
    const int key = k0w + l16, kc_row = min(key, N - 1);
    const float c = LOG2E * 0.125f;
    const float lam = lambda_of(ep, bh);

    // Per-head buffer resources: rows at or beyond N read as zero.  Offsets are unsigned 32-bit: the caller checked
    // that N + 256 rows of Q1 and Q2 fit, and the workspace's dO rows (256 bytes each, N at most 2^23) do.
    const unsigned rbq1 = (unsigned)gs.n[G_Q1] * 2u, rbq2 = (unsigned)gs.n[G_Q2] * 2u;
    const unsigned n1 = (unsigned)(N - 1);
    const __amdgpu_buffer_rsrc_t rq1 = __builtin_amdgcn_make_buffer_rsrc((void*)(gq1 + gbase(G_Q1)), (short)0,
                                                                         (int)(n1 * rbq1 + D * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rq2 = __builtin_amdgcn_make_buffer_rsrc((void*)(gq2 + gbase(G_Q2)), (short)0,
                                                                         (int)(n1 * rbq2 + D * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rdo = __builtin_amdgcn_make_buffer_rsrc((void*)(gdo + hv), (short)0,
                                                                         (int)((unsigned)N * (DV * 2u)), 0x00020000);
    const __amdgpu_buffer_rsrc_t rst = __builtin_amdgcn_make_buffer_rsrc((void*)(stats + (size_t)bh * N * STAT_FLOATS),
                                                                         (short)0, N * (STAT_FLOATS * 4), 0x00020000);

    // Direct loads per wave and tile: Q1 rows 8 wave .. + 7, Q2 the same, dO rows 4 p .. 4 p + 3 for pieces
    // p = wave and wave + 4 (lane L writes position 16 L of a 1 KiB piece), and stat `wave` of the tile's 32 queries
    // (lanes 0..31, 4 bytes each, so the stats land as [stat][query]).  Loads are issued unconditionally, also for
    // tiles past the end (out of range: zeros), so every iteration issues the same number.
    const int qrow = 8 * wave + (lane >> 3);
    const unsigned q_chunk = (((lane & 7) ^ q_sw(qrow))) << 4;
    const unsigned q1_voff = (unsigned)qrow * rbq1 + q_chunk, q2_voff = (unsigned)qrow * rbq2 + q_chunk;
    const unsigned q1_step = TILE * rbq1, q2_step = TILE * rbq2;   // bytes per tile
    unsigned do_voff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 4 * (wave + WAVES * j) + (lane >> 4);
        do_voff[j] = (unsigned)r * (DV * 2) + ((((lane & 15) ^ do_sw(r))) << 4);
    }
    const unsigned st_voff = (unsigned)(lane & 31) * (STAT_FLOATS * 4) + 4u * (unsigned)wave;
    auto issue = [&](auto S, int u) __attribute__((always_inline)) {
        unsigned char* s = pick3<decltype(S)::value>(sl0, sl1, sl2);
        check_fill(s + 1024 * wave, 16);
        check_fill(s + Q_TILE_BYTES + 1024 * wave, 16);
#pragma unroll
        for (int j = 0; j < 2; ++j) check_fill(s + 2 * Q_TILE_BYTES + 1024 * (wave + WAVES * j), 16);
        if (lane < 32) check_fill(s + ST_OFF + 128 * wave, 4);   // lanes 0..31 load 4 bytes each
        check_fence();
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq1, (lds_void*)(s + 1024 * wave), 16,
                                                 (int)(q1_voff + (unsigned)u * q1_step), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq2, (lds_void*)(s + Q_TILE_BYTES + 1024 * wave), 16,
                                                 (int)(q2_voff + (unsigned)u * q2_step), 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rdo, (lds_void*)(s + 2 * Q_TILE_BYTES + 1024 * (wave + WAVES * j)),
                                                     16, (int)(do_voff[j] + (unsigned)u * (TILE * DV * 2)), 0, 0, 0);
        if (lane < 32)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rst, (lds_void*)(s + ST_OFF + 128 * wave), 4,
                                                     (int)(st_voff + (unsigned)u * (TILE * STAT_FLOATS * 4)), 0, 0, 0);
    };

    const int n_qt = (N + TILE - 1) / TILE;
    const int u_first = causal ? k0 / TILE : 0;                  // workgroup's first query tile
    const int n_iter = n_qt - u_first;
    if (n_iter > 0) issue(Slot<0>{}, u_first);
    if (n_iter > 0) issue(Slot<1>{}, u_first + 1);

    // The wave's K1, K2 and V rows as B operands (k = feature, n = key): lane holds feature 32 kh + 8 g .. + 7 of
    // key `key`.  Loaded after the first tiles' direct loads and used before the loop, so the compiler waits for
    // them there and places no wait for them inside the loop.
    bf16x8 kb1[2], kb2[2], vb[4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
        kb1[kh] = *(const bf16x8*)(gk1 + gbase(G_K1) + kc_row * gs.n[G_K1] + 32 * kh + 8 * g);
        kb2[kh] = *(const bf16x8*)(gk2 + gbase(G_K2) + kc_row * gs.n[G_K2] + 32 * kh + 8 * g);
    }
#pragma unroll
    for (int kh = 0; kh < 4; ++kh) vb[kh] = *(const bf16x8*)(gv + gbase(G_V) + kc_row * gs.n[G_V] + 32 * kh + 8 * g);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) asm volatile("" ::"v"(kb1[kh]), "v"(kb2[kh]));
#pragma unroll
    for (int kh = 0; kh < 4; ++kh) asm volatile("" ::"v"(vb[kh]));
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();

    f32x4 av[8], ak1[4], ak2[4];   // dV^T, dK1^T, dK2^T: feature 16 fb + 4 g + i, key = lane's key
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int fb = 0; fb < 8; ++fb) av[fb][i] = 0.f;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) { ak1[fb][i] = 0.f; ak2[fb][i] = 0.f; }
    }

    // Read offsets.  16-row reads (A operands of S and dP): row 16 mb + l16, logical chunk 4 kh + g; the swizzles
    // depend only on the row's low bits, so q_off(16 mb + l16, 4 kh + g) = (q_rd0 ^ 64 kh) + 2048 mb and likewise
    // for dO with 4096 mb.  Transposing reads (A operands of dV^T and dK^T): lane 4 jj + qq of 16-lane group g
    // supplies row 4 g + jj (then 16 + 4 g + jj), features 16 fb + 4 qq .. + 3; feature block fb XORs 32 fb into
    // the offset.
    const int q_rd0 = q_off(l16, g), do_rd0 = do_off(l16, g);
    const int jj = (lane >> 2) & 3, qq = lane & 3;
    const int q_tr0 = q_off(4 * g + jj, qq >> 1) + 8 * (qq & 1);
    const int do_tr0 = do_off(4 * g + jj, qq >> 1) + 8 * (qq & 1);
    auto tr_frag = [&](const unsigned char* p, int step) __attribute__((always_inline)) {
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + step));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    auto step = [&](auto S, int j) __attribute__((always_inline)) {   // S = j % 4
        constexpr int s0 = decltype(S)::value;
        const int u = u_first + j;
        issue(Slot<(s0 + 2) % 3>{}, u + 2);
        if (!causal || u * TILE + TILE - 1 >= k0w) {
            const unsigned char* sb = pick3<s0>(sl0, sl1, sl2);
            const unsigned char* q1s = sb;
            const unsigned char* q2s = sb + Q_TILE_BYTES;
            const unsigned char* dos = sb + 2 * Q_TILE_BYTES;
            const float* sts = (const float*)(sb + ST_OFF);
            __builtin_amdgcn_s_setprio(1);
            f32x4 s1[2], s2[2], dp[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) { s1[mb][i] = 0.f; s2[mb][i] = 0.f; dp[mb][i] = 0.f; }
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const int off = (q_rd0 ^ (64 * kh)) + 2048 * mb;
                    s1[mb] = mfma16(*(const bf16x8*)(q1s + off), kb1[kh], s1[mb]);
                    s2[mb] = mfma16(*(const bf16x8*)(q2s + off), kb2[kh], s2[mb]);
                }
#pragma unroll
                for (int kh = 0; kh < 4; ++kh)
                    dp[mb] = mfma16(*(const bf16x8*)(dos + (do_rd0 ^ (64 * kh)) + 4096 * mb), vb[kh], dp[mb]);
            }
            __builtin_amdgcn_s_setprio(0);
            const bool edge = (causal && u * TILE < k0w + KW - 1) || u * TILE + TILE > N;
            float w[8], g1[8], g2[8];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int qo = 16 * mb + 4 * g;   // first of the lane's 4 queries in block mb
                const f32x4 L1 = *(const f32x4*)(sts + 0 * TILE + qo), L2 = *(const f32x4*)(sts + 1 * TILE + qo);
                const f32x4 E1 = *(const f32x4*)(sts + 2 * TILE + qo), E2 = *(const f32x4*)(sts + 3 * TILE + qo);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int x = 4 * mb + i;
                    const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[mb][i], c, -L1[i]));
                    const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[mb][i], c, -L2[i]));
                    w[x] = a - lam * b;
                    g1[x] = a * (dp[mb][i] - E1[i]);
                    g2[x] = b * (dp[mb][i] - E2[i]);   // times -lambda at the end
                }
            }
            if (edge) {
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const int qr = u * TILE + 16 * (x >> 2) + 4 * g + (x & 3);
                    const bool vis = qr < N && (!causal || key <= qr);
                    w[x] = vis ? w[x] : 0.f;
                    g1[x] = vis ? g1[x] : 0.f;
                    g2[x] = vis ? g2[x] : 0.f;
                }
            }
            u32x4 xw, x1, x2;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                xw[k] = pack2(w[2 * k], w[2 * k + 1]);
                x1[k] = pack2(g1[2 * k], g1[2 * k + 1]);
                x2[k] = pack2(g2[2 * k], g2[2 * k + 1]);
            }
            const bf16x8 pw = __builtin_bit_cast(bf16x8, xw), p1 = __builtin_bit_cast(bf16x8, x1),
                         p2 = __builtin_bit_cast(bf16x8, x2);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int fb = 0; fb < 8; ++fb) av[fb] = mfma16(tr_frag(dos + (do_tr0 ^ (32 * fb)), 16 * 256), pw, av[fb]);
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
                ak1[fb] = mfma16(tr_frag(q1s + (q_tr0 ^ (32 * fb)), 16 * 128), p1, ak1[fb]);
                ak2[fb] = mfma16(tr_frag(q2s + (q_tr0 ^ (32 * fb)), 16 * 128), p2, ak2[fb]);
            }
            __builtin_amdgcn_s_setprio(0);
        }
        // The loads of this iteration (tile u + 2, into the slot tile u - 1 left) may stay in flight past the
        // barrier; tile u + 1 has landed.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(DKDV_LOADS));
        lds_barrier();
    };
    for (int j = 0; j < n_iter; j += 3) {
        step(Slot<0>{}, j);
        if (j + 1 < n_iter) step(Slot<1>{}, j + 1);
        if (j + 2 < n_iter) step(Slot<2>{}, j + 2);
    }
    // Drain the trailing prefetches before the workgroup can retire (their LDS writes must not outlive it).
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    if (key >= N) return;
    const float sc1 = 0.125f, sc2 = -lam * 0.125f;
    uint16_t* r1 = dk1 + gbase(G_DK1) + key * gs.n[G_DK1] + 4 * g;
    uint16_t* r2 = dk2 + gbase(G_DK2) + key * gs.n[G_DK2] + 4 * g;
    uint16_t* rvv = dv + gbase(G_DV) + key * gs.n[G_DV] + 4 * g;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
        u32x2 w1, w2;
        w1[0] = pack2(ak1[fb][0] * sc1, ak1[fb][1] * sc1);
        w1[1] = pack2(ak1[fb][2] * sc1, ak1[fb][3] * sc1);
        w2[0] = pack2(ak2[fb][0] * sc2, ak2[fb][1] * sc2);
        w2[1] = pack2(ak2[fb][2] * sc2, ak2[fb][3] * sc2);
        *(u32x2*)(r1 + 16 * fb) = w1;
        *(u32x2*)(r2 + 16 * fb) = w2;
    }
#pragma unroll
    for (int fb = 0; fb < 8; ++fb) {
        u32x2 wv;
        wv[0] = pack2(av[fb][0], av[fb][1]);
        wv[1] = pack2(av[fb][2], av[fb][3]);
        *(u32x2*)(rvv + 16 * fb) = wv;
    }
}

// ---------------------------------------------------------------------------------------------------------------
// 4. dlambda: one workgroup per head, fixed summation order.
// ---------------------------------------------------------------------------------------------------------------
constexpr int DL_THREADS = 1024;
constexpr int DL_UNROLL = 4;
static_assert(DL_UNROLL == 4, "the per-thread total below adds four accumulators");
__global__ __launch_bounds__(DL_THREADS) void bwd_dlambda_kernel(const float* __restrict__ dl_rows,
                                                                 float* __restrict__ dlambda, int B, int H, int N) {
    __shared__ float red[DL_THREADS];
    const int hh = blockIdx.x, tid = threadIdx.x;
    // Each thread sums a fixed subset of the head's B x N row shares in a fixed order, with DL_UNROLL independent
    // accumulators so that as many loads are in flight; then a fixed-shape tree over the threads.
    float acc[DL_UNROLL];
#pragma unroll
    for (int k = 0; k < DL_UNROLL; ++k) acc[k] = 0.f;
    for (int b = 0; b < B; ++b) {
        const float* p = dl_rows + ((size_t)b * H + hh) * N;
        int i = tid;
        for (; i + (DL_UNROLL - 1) * DL_THREADS < N; i += DL_UNROLL * DL_THREADS)
#pragma unroll
            for (int k = 0; k < DL_UNROLL; ++k) acc[k] += p[i + k * DL_THREADS];
        for (; i < N; i += DL_THREADS) acc[0] += p[i];
    }
    red[tid] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    __syncthreads();
    for (int s = DL_THREADS / 2; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    if (tid == 0) dlambda[hh] = red[0];
}

}  // namespace

size_t bwd_bf16_workspace_bytes(int64_t BH, int64_t N) {
    const size_t rows = (size_t)BH * (size_t)N;
    // dO (bf16, 2d per row) | stats (4 floats per row) | dlambda shares (1 float per row), each 256-byte aligned
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return up(rows * DV * 2) + up(rows * STAT_FLOATS * 4) + up(rows * 4);
}

hipError_t launch_bwd_bf16_d64(const uint16_t* q1, const uint16_t* k1, const uint16_t* q2, const uint16_t* k2,
                               const uint16_t* v, const uint16_t* dy, const float* saved, uint16_t* dq1,
                               uint16_t* dk1, uint16_t* dq2, uint16_t* dk2, uint16_t* dv, float* dlambda, int64_t B,
                               int64_t H, int64_t N, int causal, Epilogue ep, const BwdStrides& gs, void* workspace,
                               hipStream_t stream) {
    const int64_t BH = B * H, rows = BH * N;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    unsigned char* ws = (unsigned char*)workspace;
    uint16_t* dO = (uint16_t*)ws;
    float* stats = (float*)(ws + up((size_t)rows * DV * 2));
    float* dl_rows = (float*)(ws + up((size_t)rows * DV * 2) + up((size_t)rows * STAT_FLOATS * 4));
    const int64_t pre_blocks = (rows + PRE_ROWS - 1) / PRE_ROWS;
    const int n_blocks = (int)((N + BLOCK - 1) / BLOCK);
    const int64_t grid = (int64_t)n_blocks * BH;
    const int64_t kv_grid = (int64_t)((N + KBLK - 1) / KBLK) * BH;
    if (pre_blocks > 0x7fffffff || grid > 0x7fffffff || kv_grid > 0x7fffffff) return hipErrorInvalidValue;
    if (rows == 0) {   // only dlambda (zeros)
        hipLaunchKernelGGL(bwd_dlambda_kernel, dim3((unsigned)H), dim3(DL_THREADS), 0, stream, dl_rows, dlambda,
                           (int)B, (int)H, 0);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)pre_blocks), dim3(THREADS), 0, stream, dy, saved, dO, stats,
                       dl_rows, rows, (int)N, (int)H, gs, ep);
    // Group sizes for the grid order (xcd_head_group); a block's fixed cost taken as 1.5 of the units by which
    // consecutive blocks' work differs, as measured for the forward's row tiles.  dQ runs two workgroups per CU,
    // dK/dV three.
    const int xg_q = xcd_head_group(BH, n_blocks, causal, 1.5, 64);
    const int xg_kv = xcd_head_group(BH, (N + KBLK - 1) / KBLK, causal, 1.5, 96);
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)grid), dim3(THREADS), 0, stream, q1, k1, q2, k2, v, dO, stats,
                       dq1, dq2, (int)BH, (int)N, n_blocks, causal ? 1 : 0, (int)H, gs, ep, xg_q);
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)kv_grid), dim3(THREADS), 0, stream, q1, k1, q2, k2, v, dO,
                       stats, dk1, dk2, dv, (int)BH, (int)N, causal ? 1 : 0, (int)H, gs, ep, xg_kv);
    hipLaunchKernelGGL(bwd_dlambda_kernel, dim3((unsigned)H), dim3(DL_THREADS), 0, stream, dl_rows, dlambda, (int)B,
                       (int)H, (int)N);
    return hipGetLastError();
}

}  // namespace diffattn
