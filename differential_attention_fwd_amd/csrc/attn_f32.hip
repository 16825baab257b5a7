// fp32 differential attention (d = 8 or 64, 2d-wide values), any Nq <= Nk, end-aligned causal mask.
//
// Operation (Ultralytics glossary "Differential Transformer", section on how differential attention works: worked
// example and the paragraph after it): two softmax maps of q1.k1/sqrt(d) and q2.k2/sqrt(d) over the visible keys,
// output sum_j (a_j - lambda b_j) v_j, then optionally the per-head RMS normalisation and (1 - lambda_init) scale.
//
// This is the full-precision path (the pages' own example runs in fp32).  It is not the throughput path: one
// workgroup per query row evaluates each softmax exactly in three sweeps over the keys (maximum, sum, weighted
// value sum), recomputing the scores each sweep, so it holds no per-key state beyond one 256-key chunk in LDS.
#include "launch.h"

namespace diffattn {
namespace {

constexpr int THREADS = 256;
constexpr int MAX_DV = 128;

__device__ __forceinline__ float block_max(float x, float* red) {
    for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum(float x, float* red) {
    for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ __forceinline__ float dotf(const float* __restrict__ a, const float* __restrict__ b, int d) {
    float acc = 0.f;
    for (int t = 0; t < d; ++t) acc = __builtin_fmaf(a[t], b[t], acc);
    return acc;
}

__global__ __launch_bounds__(THREADS) void attn_f32_kernel(const float* __restrict__ q1, const float* __restrict__ k1,
                                                           const float* __restrict__ q2, const float* __restrict__ k2,
                                                           const float* __restrict__ v, float* __restrict__ out,
                                                           int64_t Nq, int64_t Nk, int d, int causal, Epilogue ep) {
    __shared__ float w[THREADS];
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;  // flattened [BH][Nq]
    const int64_t bh = row / Nq, i = row % Nq;
    const int64_t nvis = causal ? min(Nk, i + (Nk - Nq) + 1) : Nk;
    const int dv = 2 * d;
    const float* qa = q1 + row * d;
    const float* qb = q2 + row * d;
    const float* ka = k1 + bh * Nk * d;
    const float* kb = k2 + bh * Nk * d;
    const float* vv = v + bh * Nk * dv;
    const float root_d = sqrtf((float)d);
    const float lam = lambda_of(ep, (int)bh);

    float mx1 = -INFINITY, mx2 = -INFINITY;
    for (int64_t j = tid; j < nvis; j += THREADS) {
        mx1 = fmaxf(mx1, dotf(qa, ka + j * d, d) / root_d);
        mx2 = fmaxf(mx2, dotf(qb, kb + j * d, d) / root_d);
    }
    const float m1 = block_max(mx1, red);
    const float m2 = block_max(mx2, red);
    float z1 = 0.f, z2 = 0.f;
    for (int64_t j = tid; j < nvis; j += THREADS) {
        z1 += expf(dotf(qa, ka + j * d, d) / root_d - m1);
        z2 += expf(dotf(qb, kb + j * d, d) / root_d - m2);
    }
    const float s1 = block_sum(z1, red);
    const float s2 = block_sum(z2, red);

    float o = 0.f;
    for (int64_t j0 = 0; j0 < nvis; j0 += THREADS) {
        const int64_t j = j0 + tid;
        __syncthreads();
        if (j < nvis) {
            const float a = expf(dotf(qa, ka + j * d, d) / root_d - m1) / s1;
            const float b = expf(dotf(qb, kb + j * d, d) / root_d - m2) / s2;
            w[tid] = a - lam * b;
        }
        __syncthreads();
        if (tid < dv) {
            const int64_t cnt = min((int64_t)THREADS, nvis - j0);
            for (int64_t t = 0; t < cnt; ++t) o = __builtin_fmaf(w[t], vv[(j0 + t) * dv + tid], o);
        }
    }
    if (ep.normalise) {
        const float ss = block_sum(tid < dv ? o * o : 0.f, red);
        o = o / sqrtf(ss / (float)dv + 1e-5f) * ep.out_scale;
    }
    if (tid < dv) out[row * dv + tid] = o;
}

}  // namespace

hipError_t launch_attn_f32(const float* q1, const float* k1, const float* q2, const float* k2, const float* v,
                           float* out, int64_t BH, int64_t Nq, int64_t Nk, int d, int causal, Epilogue ep,
                           hipStream_t stream) {
    const int64_t blocks = BH * Nq;
    if (blocks > 0x7fffffff || 2 * d > MAX_DV) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)blocks), dim3(THREADS), 0, stream, q1, k1, q2, k2, v, out, Nq,
                       Nk, d, causal ? 1 : 0, ep);
    return hipGetLastError();
}

}  // namespace diffattn
