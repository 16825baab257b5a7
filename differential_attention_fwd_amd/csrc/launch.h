// Internal launcher declarations shared by the C-ABI layer and the kernel translation units.
// Every launcher assumes its arguments were validated by the ABI layer and only enqueues work on `stream`;
// it returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

// Per-call epilogue parameters: raw output (layer 0) or RMS-normalised and scaled by (1 - lambda_init).
struct Epilogue {
    float lambda;                // weight of the second softmax map (when lambda_heads is null)
    int normalise;               // 0: raw (map1 - lambda map2) V; 1: RMS norm (eps 1e-5, no affine) then * out_scale
    float out_scale;             // 1 - lambda_init(layer) when normalise
    const float* lambda_heads;   // optional device array: lambda of head h is lambda_heads[h] (overrides lambda)
    int heads;                   // H, to find a (batch, head) unit's head: h = bh % heads
};

// The lambda of (batch, head) unit bh.
__device__ __forceinline__ float lambda_of(const Epilogue& ep, int bh) {
    return ep.lambda_heads ? ep.lambda_heads[bh % ep.heads] : ep.lambda;
}

// Training statistics of one query row (d = 64), written by the forward for the backward pass, fp32:
//   [0] lse1, [1] lse2: log-sum-exp of each map in log2 units of the scaled scores (p = 2^(s log2(e)/sqrt(d) - lse))
//   [2] r = 1 / sqrt(mean(o^2) + 1e-5) of the combined row o (1 when the layer is not normalised), [3] unused
//   [SAVED_O1 ..] o1 = map 1 times V (128 floats), [SAVED_O2 ..] o2 = map 2 times V (128 floats).
constexpr int SAVED_O1 = 4;
constexpr int SAVED_O2 = 4 + 128;
constexpr int SAVED_FLOATS = 4 + 256;   // 1040 bytes per row

// Element strides of the six prefill tensors, indexed q1, k1, q2, k2, v, out: batch, head and row.  The feature
// dimension is contiguous.
struct Strides {
    int64_t b[6], h[6], n[6];
};
enum { S_Q1 = 0, S_K1 = 1, S_Q2 = 2, S_K2 = 3, S_V = 4, S_OUT = 5 };

// Dense [B][H][N][d] (and [B][H][N][2d] for v and out) strides.
inline Strides contiguous_strides(int64_t H, int64_t N, int64_t d) {
    Strides s;
    for (int k = 0; k < 6; ++k) {
        const int64_t w = (k == S_V || k == S_OUT) ? 2 * d : d;
        s.b[k] = H * N * w;
        s.h[k] = N * w;
        s.n[k] = w;
    }
    return s;
}

// bf16 prefill, d = 64, 2d = 128: fused one-pass kernel (two online softmaxes, two MFMA accumulators).  With a
// non-null `saved` ([BH][N][SAVED_FLOATS] fp32) it also writes each row's training statistics.  The caller has
// checked that every head's K and V rows, N + 256 of them, span less than 4 GiB (32-bit buffer offsets).
hipError_t launch_prefill_bf16_d64(const uint16_t* q1, const uint16_t* k1, const uint16_t* q2, const uint16_t* k2,
                                   const uint16_t* v, uint16_t* out, int64_t B, int64_t H, int64_t N, int causal,
                                   const Strides& st, Epilogue ep, float* saved, hipStream_t stream);

// Partial state of one row over one key range, the split launches' workspace format (the decode and the split-key
// prefill), PARTIAL_FLOATS fp32: [0] m1, [2] m2 the two maps' offsets (log2 units of the scaled scores, -inf for a
// row that saw no key), [1] l1, [3] l2 their sums at those offsets, then the unnormalised O1 and O2 (128 each).
constexpr int PARTIAL_FLOATS = 4 + 2 * 128;

// Log-sum-exp merge of the n partial states at `part` (consecutive, PARTIAL_FLOATS apart) of one row, in one wave:
// lane owns channels 2 lane and 2 lane + 1 of O1 and O2.  The maxima are taken with the lanes striding over the
// states; the sums then run over the states in order, eight states' loads in flight at a time.  M1 or M2 is -inf
// only when no state holds a key for that map (then every weight is taken against 0, and the sums stay 0).
struct MergedRow {
    float M1, M2, L1, L2, o1a, o1b, o2a, o2b;
};
__device__ __forceinline__ MergedRow merge_states(const float* __restrict__ part, int n, int lane) {
    typedef float f32x4m __attribute__((ext_vector_type(4)));
    typedef float f32x2m __attribute__((ext_vector_type(2)));
    float m1 = -INFINITY, m2 = -INFINITY;
    for (int s = lane; s < n; s += 64) {
        m1 = fmaxf(m1, part[s * PARTIAL_FLOATS + 0]);
        m2 = fmaxf(m2, part[s * PARTIAL_FLOATS + 2]);
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) {
        m1 = fmaxf(m1, __shfl_xor(m1, x));
        m2 = fmaxf(m2, __shfl_xor(m2, x));
    }
    MergedRow r{m1, m2, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float b1 = m1 == -INFINITY ? 0.f : m1, b2 = m2 == -INFINITY ? 0.f : m2;
    auto add = [&](const f32x4m& hd, const f32x2m& a, const f32x2m& b) {
        const float w1 = __builtin_amdgcn_exp2f(hd[0] - b1);
        const float w2 = __builtin_amdgcn_exp2f(hd[2] - b2);
        r.L1 += w1 * hd[1];
        r.L2 += w2 * hd[3];
        r.o1a += w1 * a[0];
        r.o1b += w1 * a[1];
        r.o2a += w2 * b[0];
        r.o2b += w2 * b[1];
    };
    int s = 0;
    constexpr int IN_FLIGHT = 8;
    for (; s + IN_FLIGHT <= n; s += IN_FLIGHT) {
        f32x4m hd[IN_FLIGHT];
        f32x2m a[IN_FLIGHT], b[IN_FLIGHT];
#pragma unroll
        for (int u = 0; u < IN_FLIGHT; ++u) {
            const float* p = part + (s + u) * PARTIAL_FLOATS;
            hd[u] = *(const f32x4m*)p;
            a[u] = *(const f32x2m*)(p + 4 + 2 * lane);
            b[u] = *(const f32x2m*)(p + 4 + 128 + 2 * lane);
        }
#pragma unroll
        for (int u = 0; u < IN_FLIGHT; ++u) add(hd[u], a[u], b[u]);
    }
    for (; s < n; ++s) {
        const float* p = part + s * PARTIAL_FLOATS;
        add(*(const f32x4m*)p, *(const f32x2m*)(p + 4 + 2 * lane), *(const f32x2m*)(p + 4 + 128 + 2 * lane));
    }
    return r;
}

// The n states merged into one state of the same format at `dst` (a level of a merge tree).
__device__ __forceinline__ void merge_partial_state(const float* __restrict__ part, int n, float* __restrict__ dst,
                                                    int lane) {
    typedef float f32x2m __attribute__((ext_vector_type(2)));
    const MergedRow r = merge_states(part, n, lane);
    if (lane == 0) {
        dst[0] = r.M1;
        dst[1] = r.L1;
        dst[2] = r.M2;
        dst[3] = r.L2;
    }
    *(f32x2m*)(dst + 4 + 2 * lane) = f32x2m{r.o1a, r.o1b};
    *(f32x2m*)(dst + 4 + 128 + 2 * lane) = f32x2m{r.o2a, r.o2b};
}

// The n states merged, the epilogue of (batch, head) unit bh applied, and the row's 128 outputs stored in bf16.
// At least one state must hold a key for each map.
__device__ __forceinline__ void merge_partial_row(const float* __restrict__ part, int n, const Epilogue& ep, int bh,
                                                  uint16_t* __restrict__ out_row, int lane) {
    const MergedRow r = merge_states(part, n, lane);
    const float inv1 = 1.f / r.L1, inv2 = lambda_of(ep, bh) / r.L2;
    float ya = r.o1a * inv1 - r.o2a * inv2;
    float yb = r.o1b * inv1 - r.o2b * inv2;
    if (ep.normalise) {
        float ss = ya * ya + yb * yb;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
        const float rr = __builtin_amdgcn_rsqf(ss * (1.f / 128) + 1e-5f) * ep.out_scale;
        ya *= rr;
        yb *= rr;
    }
    const unsigned w = (unsigned)__builtin_bit_cast(unsigned short, (__bf16)ya) |
                       ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)yb) << 16);
    *(unsigned*)(out_row + 2 * lane) = w;
}

// Grid order for launches of many (block, head) items, heaviest block first.  The hardware deals workgroups to the
// 8 XCDs in turn, so with 8 | B*H the plain order (r = bid / BH, bh = bid % BH) gives XCD x the heads bh = x
// (mod 8), all of them at once.  With a group size g > 0, XCD x takes its heads g at a time instead (all blocks of
// a group, heaviest first, before the next group), so fewer heads' K and V (or Q and dO) compete for its 4 MiB L2.
// Workgroup bid's item: r = 0 for the heaviest block, and its (batch, head) unit bh.
__device__ __forceinline__ void xcd_item(int bid, int BH, int R, int g, int& r, int& bh) {
    if (g > 0) {
        const int x = bid & 7, i = bid >> 3;
        const int per_group = g * R;
        const int q = i / per_group, rem = i - q * per_group;
        r = rem / g;
        bh = 8 * (q * g + rem - r * g) + x;
    } else {
        r = bid / BH;
        bh = bid % BH;
    }
}
// The group size for BH heads of R blocks each (0: the plain order): the smallest divisor of the XCD's head count
// BH / 8 whose modelled schedule ends within 0.5% of the plain order's.  The model dispatches the XCD's items in
// grid order to whichever of its `slots` workgroup slots (workgroups per CU x 32 CUs) frees first; block r costs
// fixed_units + (R - r) units when causal (the heaviest first), fixed_units + R otherwise, a unit being the work
// that shrinks from one block to the next.
int xcd_head_group(int64_t BH, int64_t R, int causal, double fixed_units, int slots);

// Split-key prefill for launches too small to fill the GPU (see prefill_key_splits): each row tile's key range is
// cut into splits handled by separate workgroups, which write per-row partial states; a merge kernel then combines
// each row's non-empty ones and applies the epilogue.
// Key splits per row tile for a dense (B*H, N) prefill (1: the ordinary launch is the faster).
int prefill_key_splits(int64_t BH, int64_t N, int causal);
// The largest prefill_key_splits over both masks, which sizes the workspace.
int prefill_key_splits_max(int64_t BH, int64_t N);
// The dense bf16 prefill (d = 64, as launch_prefill_bf16_d64 with contiguous strides) through key splits: `part`
// holds B*H*N*prefill_key_splits_max(B*H, N)*PARTIAL_FLOATS floats (unused when the plan is 1 split).
hipError_t launch_prefill_split_bf16_d64(const uint16_t* q1, const uint16_t* k1, const uint16_t* q2,
                                         const uint16_t* k2, const uint16_t* v, uint16_t* out, int64_t B, int64_t H,
                                         int64_t N, int causal, Epilogue ep, float* part, hipStream_t stream);

// Element strides of the backward's caller tensors, indexed q1, k1, q2, k2, v, dy, dq1, dk1, dq2, dk2, dv: batch,
// head and row.  The feature dimension is contiguous.
constexpr int BWD_TENSORS = 11;
struct BwdStrides {
    int64_t b[BWD_TENSORS], h[BWD_TENSORS], n[BWD_TENSORS];
};
enum { G_Q1 = 0, G_K1, G_Q2, G_K2, G_V, G_DY, G_DQ1, G_DK1, G_DQ2, G_DK2, G_DV };

// Dense [B][H][N][d] (and [B][H][N][2d] for v, dy and dv) strides.
inline BwdStrides dense_bwd_strides(int64_t H, int64_t N, int64_t d) {
    BwdStrides s;
    for (int k = 0; k < BWD_TENSORS; ++k) {
        const int64_t w = (k == G_V || k == G_DY || k == G_DV) ? 2 * d : d;
        s.b[k] = H * N * w;
        s.h[k] = N * w;
        s.n[k] = w;
    }
    return s;
}

// bf16 backward, d = 64: preprocess, dQ, dK/dV and dlambda kernels (see backward_bf16.hip).  `saved` is the
// training forward's [BH][N][SAVED_FLOATS]; `workspace` holds bwd_bf16_workspace_bytes(BH, N) bytes (256-byte
// aligned); dlambda receives H floats (per head, summed over the batch).  Caller tensors are addressed through `gs`;
// the caller has checked that every head's Q1, K1, Q2, K2 and V rows, N + 256 of them, span less than 4 GiB.
size_t bwd_bf16_workspace_bytes(int64_t BH, int64_t N);
hipError_t launch_bwd_bf16_d64(const uint16_t* q1, const uint16_t* k1, const uint16_t* q2, const uint16_t* k2,
                               const uint16_t* v, const uint16_t* dy, const float* saved, uint16_t* dq1,
                               uint16_t* dk1, uint16_t* dq2, uint16_t* dk2, uint16_t* dv, float* dlambda, int64_t B,
                               int64_t H, int64_t N, int causal, Epilogue ep, const BwdStrides& gs, void* workspace,
                               hipStream_t stream);

// fp32 path (d = 8 or 64), general Nq <= Nk with end-aligned causal mask; exact three-pass softmax per row.
hipError_t launch_attn_f32(const float* q1, const float* k1, const float* q2, const float* k2, const float* v,
                           float* out, int64_t BH, int64_t Nq, int64_t Nk, int d, int causal, Epilogue ep,
                           hipStream_t stream);

// bf16 decode, d = 64: split kernel writing per-split partial states, then the merge + epilogue kernel.
// T new tokens per (b, h) (1 <= T <= 16; queries [BH][T][d], out [BH][T][2d]); caches [BH][L][...]; lens: optional
// device array of B cache lengths (clamped on the device to [T, L]), with b = bh / H.
// Paged decode caches: the rows of sequence b live in pages of 2^log2_page rows in pools [num_pages][H][page][w];
// logical row r of sequence b is row r % page of page table[b * max_pages + r / page] (entries clamped to
// [0, num_pages)).  L = max_pages * page.
struct DecodePages {
    const int* table;
    int max_pages, log2_page, num_pages;
};

// Element strides of the three padded decode caches, indexed k1, k2, v: batch, head and row.  The feature dimension
// is contiguous.  Paged caches ignore them.
struct CacheStrides {
    int64_t b[3], h[3], n[3];
};
enum { C_K1 = 0, C_K2 = 1, C_V = 2 };

// Dense [B][H][L][d] (and [B][H][L][2d] for v) strides.
inline CacheStrides dense_cache_strides(int64_t H, int64_t L, int64_t d) {
    CacheStrides s;
    for (int k = 0; k < 3; ++k) {
        const int64_t w = k == C_V ? 2 * d : d;
        s.b[k] = H * L * w;
        s.h[k] = L * w;
        s.n[k] = w;
    }
    return s;
}

// Workspace bytes of a decode call; `ragged`: the call may pass a length array, which for some shapes selects the
// balanced plan (its states per item may exceed the fixed plan's).
size_t decode_bf16_workspace_bytes(int64_t BH, int64_t H, int64_t L, int T, bool ragged);
// pages == nullptr: padded caches addressed through cs (cache row r of head (b, h) of tensor t at element
// b cs.b[t] + h cs.h[t] + r cs.n[t]); otherwise the page pools.
hipError_t launch_decode_bf16_d64(const uint16_t* q1, const uint16_t* k1, const uint16_t* q2, const uint16_t* k2,
                                  const uint16_t* v, uint16_t* out, int64_t BH, int64_t H, int64_t L, int T,
                                  const int* lens, const DecodePages* pages, const CacheStrides& cs, Epilogue ep,
                                  void* workspace, hipStream_t stream);

}  // namespace diffattn
