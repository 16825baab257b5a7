// Fused one-pass differential attention prefill for gfx950 (bf16 in/out, fp32 accumulation, d = 64, 2d = 128).
//
// Operation (Ultralytics glossary "Differential Transformer", section on how differential attention works: worked
// example and the paragraph after it): per head and query row i, two softmax maps over the visible keys with
// scores q1.k1/sqrt(d) and q2.k2/sqrt(d), output sum_j (a_j - lambda b_j) v_j, then optionally the per-head RMS
// normalisation and the (1 - lambda_init) scale.
//
// Design (one pass over K1/K2/V, nothing N x N ever materialised):
//   * A workgroup of 4 waves owns 128 query rows of one (batch, head); each wave owns 32 rows.  Key/value tiles of
//     32 keys (K1 4 KiB, K2 4 KiB, V 8 KiB) are double-buffered through LDS.  K rows go straight from global
//     memory to LDS (global_load_lds_dwordx4, no registers); V goes through registers and is stored TRANSPOSED
//     (channel-major) so that every MFMA operand is fetched with 128-bit LDS reads.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in
//     registers).  In the accumulator layout every lane owns ONE query row (lane % 32) and 16 of the 32 keys, so
//     row statistics need only the lane pair (l, l ^ 32), exchanged with v_permlane32_swap.
//   * P^T stays in registers and feeds O^T = V^T P^T directly as the MFMA B operand.  The k-order of that product
//     is the accumulator's key order; the transposed V tile stores keys in that order, so the A operand of each
//     MFMA is one contiguous 16-byte read.  O^T's layout gives each lane one query row again, so the
//     online-softmax rescale of O is lane-local.
//   * Two online softmaxes run side by side (running max and sum per map, two O accumulators).  The running max
//     only moves when a row's new maximum exceeds it by more than 2^8 (wave-uniform decision), so the O rescale
//     is rare; exponents use exp2 with log2(e)/sqrt(d) folded into one FMA.  Map 2's exponentials are issued
//     between map 1's value MFMAs so the VALU and the matrix cores of a wave overlap.
//   * Epilogue: O1/l1 - lambda O2/l2, RMS over the 128 channels (pair-reduced), scale, bf16 round-to-nearest-even.
//   * Causal: row tiles are launched heaviest first; tiles wholly above a wave's rows are skipped by that wave,
//     and only diagonal or ragged-tail tiles pay for masking.
//
// This translation unit is compiled with -fno-honor-nans: no NaN can arise (inputs are finite, masked scores are
// -inf, and every processed row has a visible key in its first tile), and it lets v_max3 run without quieting.
#include "launch.h"

namespace diffattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int D = 64;
constexpr int DV = 128;
constexpr int BM = 128;                         // query rows per workgroup
constexpr int BN = 32;                          // keys per tile
constexpr int THREADS = 256;
constexpr int K_TILE_BYTES = BN * D * 2;        // 4 KiB
constexpr int V_TILE_BYTES = BN * DV * 2;       // 8 KiB
constexpr int STAGE_BYTES = 2 * K_TILE_BYTES + V_TILE_BYTES;
constexpr float RESCALE_THRESHOLD = 8.0f;       // log2 units: p never exceeds 2^8 between rescales
constexpr float LOG2E = 1.4426950408889634f;

// K tile: row r (key) of 128 bytes = 8 chunks of 16 bytes; chunk c lives at position c ^ ((r >> 1) & 7).  A wave's
// 16-lane read group (16 rows, one chunk) and the contiguous direct loads both touch 16 distinct bank quads.
__device__ __forceinline__ int k_off(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Transposed V tile: 128 channel rows of 64 bytes (32 keys).  Keys are stored in the accumulator's key order:
// key 16s + 8a + 4h + j sits at position 16s + 8h + 4a + j (bits 2 and 3 swapped).  Channel c occupies physical
// row (c & ~3) | ((c & 3) ^ ((c >> 4) & 1)) and its 16-byte chunk q sits at q ^ ((c >> 2) & 3): the 16
// consecutive channels of a 128-bit read group hit 16 distinct bank quads, and a transposing write group
// (4 key groups x 8 channel groups) at most 2-way shares one.  The swizzle uses only channel bits 0..4, so the
// four 32-channel blocks of a read differ by a constant offset.
__device__ __forceinline__ int vt_off(int c, int chunk) {
    const int prow = (c & ~3) | ((c & 3) ^ ((c >> 4) & 1));
    return prow * 64 + ((chunk ^ ((c >> 2) & 3)) << 4);
}
__device__ __forceinline__ int key_pos(int key) { return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1); }

// Combine a per-lane value with the value of lane (l ^ 32).
__device__ __forceinline__ float pair_max(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ unsigned pack2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float max16(const f32x16& s) {
    const float a = fmaxf(fmaxf(s[0], s[1]), s[2]), b = fmaxf(fmaxf(s[3], s[4]), s[5]);
    const float c = fmaxf(fmaxf(s[6], s[7]), s[8]), d = fmaxf(fmaxf(s[9], s[10]), s[11]);
    const float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
    return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), s[15]));
}

// Move the running max of one map if the tile's max exceeds it by more than the threshold (wave-uniform branch);
// rescales that map's O accumulator and partial sum.
__device__ __forceinline__ void update_max(const f32x16& s, float& m, float& l, f32x16 (&o)[4], float c) {
    const float m_new = fmaxf(m, pair_max(max16(s)) * c);
    if (__any(m_new > m + RESCALE_THRESHOLD)) {
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
    }
}

// p = exp2(s * c - m) for the lane's 16 keys; adds them to l and packs P^T as two bf16x8 B operands.
__device__ __forceinline__ void exp_pack(const f32x16& s, float m, float& l, float c, bf16x8& lo, bf16x8& hi) {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m));
    float t0 = (p[0] + p[1]) + (p[2] + p[3]), t1 = (p[4] + p[5]) + (p[6] + p[7]);
    float t2 = (p[8] + p[9]) + (p[10] + p[11]), t3 = (p[12] + p[13]) + (p[14] + p[15]);
    l += (t0 + t1) + (t2 + t3);
    u32x4 a, b;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        a[k] = pack2(p[2 * k], p[2 * k + 1]);
        b[k] = pack2(p[8 + 2 * k], p[8 + 2 * k + 1]);
    }
    lo = __builtin_bit_cast(bf16x8, a);
    hi = __builtin_bit_cast(bf16x8, b);
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_d64_kernel(const uint16_t* __restrict__ gq1, const uint16_t* __restrict__ gk1,
                             const uint16_t* __restrict__ gq2, const uint16_t* __restrict__ gk2,
                             const uint16_t* __restrict__ gv, uint16_t* __restrict__ gout, int BH, int N,
                             int n_row_tiles, int causal, Epilogue ep) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;     // which half of the accumulator's key rows this lane holds
    const int l32 = lane & 31;   // this lane's query row inside the wave

    // Heaviest row tiles first under the causal mask (their key range is longest).
    const int bid = blockIdx.x;
    const int rt = causal ? (n_row_tiles - 1 - bid / BH) : bid / BH;
    const int bh = bid % BH;
    const int q0 = rt * BM;
    const int q0w = q0 + wave * 32;

    const size_t head_qk = (size_t)bh * (size_t)N * D;
    const size_t head_v = (size_t)bh * (size_t)N * DV;
    // Per-head buffer resources: rows at or beyond N read as zero (and are masked), so no clamping is needed.
    // Byte sizes and offsets are unsigned 32-bit: a head's V is at most 2^23 x 256 bytes.
    const unsigned k_bytes = (unsigned)N * (D * 2u), v_bytes = (unsigned)N * (DV * 2u);
    const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc((void*)(gk1 + head_qk), (short)0, (int)k_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk2 = __builtin_amdgcn_make_buffer_rsrc((void*)(gk2 + head_qk), (short)0, (int)k_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(gv + head_v), (short)0, (int)v_bytes, 0x00020000);

    // Q fragments as the MFMA B operand: lane holds Q[q0w + l32][16 kc + 8 h .. + 7].
    bf16x8 qa[4], qb[4];
    {
        const int row = min(q0w + l32, N - 1);
        const uint16_t* p1 = gq1 + head_qk + (size_t)row * D + 8 * h;
        const uint16_t* p2 = gq2 + head_qk + (size_t)row * D + 8 * h;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            qa[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(p1 + 16 * kc));
            qb[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(p2 + 16 * kc));
        }
    }

    const int q_last = min(N, q0 + BM) - 1;
    const int n_tiles = causal ? (q_last / BN + 1) : (N + BN - 1) / BN;

    // K direct loads: wave w fills LDS bytes [1024 w, 1024 w + 1024) of each K tile, lane L position 16 L of that,
    // i.e. tile row 8 w + L / 8, stored chunk L % 8, which holds logical chunk (L % 8) ^ ((row >> 1) & 7).
    const int kd_row = 8 * wave + (lane >> 3);
    const unsigned kd_voff = kd_row * 128 + (((lane & 7) ^ ((kd_row >> 1) & 7)) << 4);
    // V loads: thread owns keys 4 kg .. 4 kg + 3 and channels 4 cg .. 4 cg + 3, with kg = lane / 8 and
    // cg = 8 wave + lane % 8 (a wave covers 32 channels of all 32 keys).
    const int kg = lane >> 3, cg = 8 * wave + (lane & 7);
    const unsigned v_voff = (4 * kg) * 256 + cg * 8;
    // Transposed store targets of the thread's 4 channels (see vt_off): channel 4 cg + i lands in physical row
    // 4 cg + (i ^ b), b = (cg >> 2) & 1, so rows i and i ^ 1 swap when b is set.
    const int vpos = key_pos(4 * kg);
    const int vt_base = vt_off(4 * cg, vpos >> 3) + (vpos & 7) * 2;  // = physical row 4 cg + b
    const int vb = (cg >> 2) & 1;
    const int vt_w0 = vt_base;                       // channel 4cg     -> row 4cg + b      (4cg+2: +128)
    const int vt_w1 = vt_base + 64 - 128 * vb;       // channel 4cg + 1 -> row 4cg + (1^b)  (4cg+3: +128)
    u32x2 st_v[4];

    auto issue_loads = [&](int t, int buf) {
        const int kv0 = t * BN;
        unsigned char* base = lds + buf * STAGE_BYTES;
        // The tile offset goes into the VGPR offset: the SGPR offset is not part of the buffer range check.
        const unsigned ko = kd_voff + (unsigned)kv0 * 128u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk1, (lds_void*)(base + 1024 * wave), 16, (int)ko, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk2, (lds_void*)(base + K_TILE_BYTES + 1024 * wave), 16, (int)ko, 0, 0,
                                                 0);
        const unsigned vo = v_voff + (unsigned)kv0 * 256u;
#pragma unroll
        for (int i = 0; i < 4; ++i) st_v[i] = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)(vo + 256u * i), 0, 0);
    };
    // Transpose the thread's 4 keys x 4 channels and store channel-major.
    auto store_v = [&](int buf) {
        unsigned char* vt = lds + buf * STAGE_BYTES + 2 * K_TILE_BYTES;
        u32x2 w[4];
        w[0][0] = __builtin_amdgcn_perm(st_v[1][0], st_v[0][0], 0x05040100u);
        w[0][1] = __builtin_amdgcn_perm(st_v[3][0], st_v[2][0], 0x05040100u);
        w[1][0] = __builtin_amdgcn_perm(st_v[1][0], st_v[0][0], 0x07060302u);
        w[1][1] = __builtin_amdgcn_perm(st_v[3][0], st_v[2][0], 0x07060302u);
        w[2][0] = __builtin_amdgcn_perm(st_v[1][1], st_v[0][1], 0x05040100u);
        w[2][1] = __builtin_amdgcn_perm(st_v[3][1], st_v[2][1], 0x05040100u);
        w[3][0] = __builtin_amdgcn_perm(st_v[1][1], st_v[0][1], 0x07060302u);
        w[3][1] = __builtin_amdgcn_perm(st_v[3][1], st_v[2][1], 0x07060302u);
        *(u32x2*)(vt + vt_w0) = w[0];
        *(u32x2*)(vt + vt_w1) = w[1];
        *(u32x2*)(vt + vt_w0 + 128) = w[2];
        *(u32x2*)(vt + vt_w1 + 128) = w[3];
    };

    // Per-lane read offsets: K A-operand (row l32, chunk 2 kc + h) and V^T A-operand (channel 32 cb + l32,
    // chunk 2 ks + h; the four channel blocks are 2 KiB apart).
    int k_rd[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) k_rd[kc] = k_off(l32, 2 * kc + h);
    const int v_rd0 = 2 * K_TILE_BYTES + vt_off(l32, h);
    const int v_rd1 = 2 * K_TILE_BYTES + vt_off(l32, 2 + h);

    f32x16 o1[4], o2[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) { o1[cb][i] = 0.f; o2[cb][i] = 0.f; }
    float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
    const float c = LOG2E * 0.125f;  // log2(e) / sqrt(64)

    issue_loads(0, 0);
    store_v(0);
    for (int t = 0; t < n_tiles; ++t) {
        __builtin_amdgcn_s_waitcnt(0);   // this thread's direct K loads and V stores of tile t are complete
        __syncthreads();
        if (t + 1 < n_tiles) issue_loads(t + 1, (t + 1) & 1);
        const int kv0 = t * BN;
        if (!causal || kv0 <= q0w + 31) {
            const unsigned char* base = lds + (t & 1) * STAGE_BYTES;
            f32x16 s1, s2;
#pragma unroll
            for (int i = 0; i < 16; ++i) { s1[i] = 0.f; s2[i] = 0.f; }
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const bf16x8 ka = *(const bf16x8*)(base + k_rd[kc]);
                const bf16x8 kb = *(const bf16x8*)(base + K_TILE_BYTES + k_rd[kc]);
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
            update_max(s1, m1, l1, o1, c);
            update_max(s2, m2, l2, o2, c);

            bf16x8 p1[2], p2[2];
            exp_pack(s1, m1, l1, c, p1[0], p1[1]);
            bf16x8 va[4][2];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) va[cb][0] = *(const bf16x8*)(base + v_rd0 + 2048 * cb);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o1[cb] = mfma(va[cb][0], p1[0], o1[cb]);
            exp_pack(s2, m2, l2, c, p2[0], p2[1]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) va[cb][1] = *(const bf16x8*)(base + v_rd1 + 2048 * cb);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o2[cb] = mfma(va[cb][0], p2[0], o2[cb]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o1[cb] = mfma(va[cb][1], p1[1], o1[cb]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) o2[cb] = mfma(va[cb][1], p2[1], o2[cb]);
        }
        if (t + 1 < n_tiles) store_v((t + 1) & 1);
    }

    // Epilogue: lane owns query row q0w + l32 and channels cb*32 + 8*(i/4) + 4h + i%4.
    l1 = pair_sum(l1);
    l2 = pair_sum(l2);
    const float inv1 = 1.f / l1;
    const float inv2 = ep.lambda / l2;
    float ss = 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float o = o1[cb][i] * inv1 - o2[cb][i] * inv2;
            o1[cb][i] = o;
            ss += o * o;
        }
    float r = 1.f;
    if (ep.normalise) {
        ss = pair_sum(ss);
        r = __builtin_amdgcn_rsqf(ss * (1.f / DV) + 1e-5f) * ep.out_scale;
    }
    const int q = q0w + l32;
    if (q < N) {
        uint16_t* orow = gout + head_v + (size_t)q * DV + 4 * h;
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
                                   const uint16_t* v, uint16_t* out, int64_t BH, int64_t N, int causal,
                                   Epilogue ep, hipStream_t stream) {
    const int n_row_tiles = (int)((N + BM - 1) / BM);
    const int64_t blocks = (int64_t)n_row_tiles * BH;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_bf16_d64_kernel, dim3((unsigned)blocks), dim3(THREADS), 0, stream, q1, k1, q2, k2, v,
                       out, (int)BH, (int)N, n_row_tiles, causal ? 1 : 0, ep);
    return hipGetLastError();
}

}  // namespace diffattn
