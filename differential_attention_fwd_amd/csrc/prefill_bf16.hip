// Fused one-pass differential attention prefill for gfx950 (bf16 in/out, fp32 accumulation, d = 64, 2d = 128).
//
// Operation (Ultralytics glossary "Differential Transformer", section on how differential attention works: worked
// example and the paragraph after it): per head and query row i, two softmax maps over the visible keys with
// scores q1.k1/sqrt(d) and q2.k2/sqrt(d), output sum_j (a_j - lambda b_j) v_j, then optionally the per-head RMS
// normalisation and the (1 - lambda_init) scale.
//
// Design (one pass over K1/K2/V, nothing N x N ever materialised):
//   * A workgroup of 4 waves owns 128 query rows of one (batch, head); each wave owns 32 rows.  Key/value tiles of
//     32 keys (K1 4 KiB, K2 4 KiB, V 8 KiB) are double-buffered through LDS with XOR-swizzled 16-byte chunks.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in
//     registers).  In the accumulator layout every lane then owns ONE query row (lane % 32) and 16 of the 32 keys,
//     so row statistics need only the lane pair (l, l ^ 32), exchanged with v_permlane32_swap.
//   * P^T stays in registers and feeds the value product O^T = V^T P^T directly as the MFMA B operand; V^T comes
//     from LDS with the transposing read ds_read_b64_tr_b16.  O^T's layout again gives each lane one query row,
//     so the online-softmax rescale of O is lane-local.
//   * Two online softmaxes run side by side (running max and sum per map, two O accumulators).  The running max
//     is only moved when a row's new maximum exceeds it by more than 2^8 (wave-uniform decision), so the O
//     rescale is rare; exponents use exp2 with log2(e)/sqrt(d) folded into one FMA.
//   * Epilogue: O1/l1 - lambda O2/l2, RMS over the 128 channels (pair-reduced), scale, bf16 round-to-nearest-even.
//   * Causal: row tiles are launched heaviest first; tiles wholly above a wave's rows are skipped by that wave,
//     and only diagonal or ragged-tail tiles pay for masking.
#include "launch.h"

namespace diffattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

// K tile: row r (key) of 128 bytes = 8 chunks of 16 bytes; chunk c lives at c ^ ((r >> 1) & 7).
__device__ __forceinline__ int k_off(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }
// V tile: row r of 256 bytes = 16 chunks; chunk c lives at c ^ (4 * (r & 3)).
__device__ __forceinline__ int v_off(int row, int chunk) { return row * 256 + ((chunk ^ ((row & 3) << 2)) << 4); }

// Combine a per-lane value with the value of lane (l ^ 32).
__device__ __forceinline__ float pair_max(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)a) |
           ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)b) << 16);
}

// One map's online-softmax step on a 32-key tile.  s: raw scores S^T (this lane: one query row, 16 keys).
// Updates the running max m (log2 units) and partial sum l, rescales o when the max moves, and returns P^T as two
// bf16x8 MFMA B operands (keys 0..15 and 16..31 of the tile, in the accumulator's key order).
__device__ __forceinline__ void softmax_step(f32x16 s, float& m, float& l, f32x16 (&o)[4], float c,
                                             bf16x8& p_lo, bf16x8& p_hi) {
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    float mx2 = fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])), fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15])));
    mx = pair_max(fmaxf(mx, mx2));
    const float m_new = fmaxf(m, mx * c);
    if (__any(m_new > m + RESCALE_THRESHOLD)) {
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
    }
    float p[16];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m));
        ps += p[i];
    }
    l += ps;
    u32x4 lo, hi;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        lo[k] = pack_bf16x2(p[2 * k], p[2 * k + 1]);
        hi[k] = pack_bf16x2(p[8 + 2 * k], p[8 + 2 * k + 1]);
    }
    p_lo = __builtin_bit_cast(bf16x8, lo);
    p_hi = __builtin_bit_cast(bf16x8, hi);
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
    const int h = lane >> 5;     // which half of the 32x32 accumulator's key rows this lane holds
    const int l32 = lane & 31;   // this lane's query row inside the wave

    // Heaviest row tiles first under the causal mask (their key range is longest).
    const int bid = blockIdx.x;
    const int rt = causal ? (n_row_tiles - 1 - bid / BH) : bid / BH;
    const int bh = bid % BH;
    const int q0 = rt * BM;
    const int q0w = q0 + wave * 32;

    const size_t head_qk = (size_t)bh * (size_t)N * D;
    const size_t head_v = (size_t)bh * (size_t)N * DV;

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

    // Cooperative tile load: K rows tid/8 (chunk tid%8); V rows tid/16 and 16 + tid/16 (chunk tid%16).
    const int kr = tid >> 3, kc_ = tid & 7;
    const int vr = tid >> 4, vc = tid & 15;
    u32x4 st_k1, st_k2, st_v0, st_v1;
    auto gload = [&](int t) {
        const int kv0 = t * BN;
        const int rk = min(kv0 + kr, N - 1);
        st_k1 = *(const u32x4*)(gk1 + head_qk + (size_t)rk * D + kc_ * 8);
        st_k2 = *(const u32x4*)(gk2 + head_qk + (size_t)rk * D + kc_ * 8);
        const int rv0 = min(kv0 + vr, N - 1), rv1 = min(kv0 + 16 + vr, N - 1);
        st_v0 = *(const u32x4*)(gv + head_v + (size_t)rv0 * DV + vc * 8);
        st_v1 = *(const u32x4*)(gv + head_v + (size_t)rv1 * DV + vc * 8);
    };
    auto lstore = [&](int buf) {
        unsigned char* base = lds + buf * STAGE_BYTES;
        *(u32x4*)(base + k_off(kr, kc_)) = st_k1;
        *(u32x4*)(base + K_TILE_BYTES + k_off(kr, kc_)) = st_k2;
        *(u32x4*)(base + 2 * K_TILE_BYTES + v_off(vr, vc)) = st_v0;
        *(u32x4*)(base + 2 * K_TILE_BYTES + v_off(vr + 16, vc)) = st_v1;
    };

    // Per-lane byte offsets of the transposing V reads (see v_off): lane supplies row 4*(g>>1) + jj of the
    // 8-key group and the 8-byte piece (qq) of 16-byte chunk 2*(g&1) + qq/2 of the 32-channel block.
    const int g = lane >> 4, jj = (lane >> 2) & 3, qq = lane & 3;
    const int vrow_lane = 4 * (g >> 1) + jj;
    const int vchunk_lo = 2 * (g & 1) + (qq >> 1);
    const int vbyte = 8 * (qq & 1);

    f32x16 o1[4], o2[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) { o1[cb][i] = 0.f; o2[cb][i] = 0.f; }
    float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
    const float c = LOG2E * 0.125f;  // log2(e) / sqrt(64)

    gload(0);
    lstore(0);
    for (int t = 0; t < n_tiles; ++t) {
        if (t + 1 < n_tiles) gload(t + 1);
        __syncthreads();
        const int kv0 = t * BN;
        if (!causal || kv0 <= q0w + 31) {
            const unsigned char* base = lds + (t & 1) * STAGE_BYTES;
            f32x16 s1, s2;
#pragma unroll
            for (int i = 0; i < 16; ++i) { s1[i] = 0.f; s2[i] = 0.f; }
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const bf16x8 ka = *(const bf16x8*)(base + k_off(l32, 2 * kc + h));
                const bf16x8 kb = *(const bf16x8*)(base + K_TILE_BYTES + k_off(l32, 2 * kc + h));
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qa[kc], s1, 0, 0, 0);
                s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qb[kc], s2, 0, 0, 0);
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
            bf16x8 p1[2], p2[2];
            softmax_step(s1, m1, l1, o1, c, p1[0], p1[1]);
            softmax_step(s2, m2, l2, o2, c, p2[0], p2[1]);

            const unsigned char* vbase = base + 2 * K_TILE_BYTES;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const int chunk = ((cb ^ jj) << 2) | vchunk_lo;
                    const int off0 = (16 * ks + vrow_lane) * 256 + (chunk << 4) + vbyte;
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + off0));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + off0 + 8 * 256));
                    const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    const bf16x8 va = __builtin_bit_cast(bf16x8, both);
                    o1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p1[ks], o1[cb], 0, 0, 0);
                    o2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p2[ks], o2[cb], 0, 0, 0);
                }
            }
        }
        if (t + 1 < n_tiles) lstore((t + 1) & 1);
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
                w[0] = pack_bf16x2(o1[cb][4 * g4 + 0] * r, o1[cb][4 * g4 + 1] * r);
                w[1] = pack_bf16x2(o1[cb][4 * g4 + 2] * r, o1[cb][4 * g4 + 3] * r);
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
