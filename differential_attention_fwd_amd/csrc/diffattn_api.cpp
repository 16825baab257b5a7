// C-ABI layer of libdiffattn.so: argument validation (before any HIP call), epilogue constants, dispatch.
// The operation and every argument's meaning are documented in include/diffattn.h.
#include "../../include/diffattn.h"

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "launch.h"

namespace {

using diffattn::Epilogue;

constexpr int ABI_VERSION = 1;

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// a * b with overflow check against a bound; returns false on overflow.
bool mul_ok(int64_t a, int64_t b, int64_t* r) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *r = a * b;
    return true;
}

// True when the strided [B][H][N][w] layout with element strides (sb, sh, sn) (feature stride 1) gives every element
// its own address, proven by ordering the dimensions of extent > 1 by stride: each stride must be at least the
// previous one times its extent (the first at least 1).  Outputs must pass: a layout that folds two elements onto one
// address would have several workgroups write it at once.  (Some exotic one-to-one layouts fail the test too; they
// are rejected rather than risked.)
bool one_to_one(int64_t B, int64_t H, int64_t N, int64_t w, int64_t sb, int64_t sh, int64_t sn) {
    int64_t st[4] = {1, sn, sh, sb}, ex[4] = {w, N, H, B};
    int n = 0;
    int64_t ds[4], de[4];
    for (int k = 0; k < 4; ++k)
        if (ex[k] > 1) { ds[n] = st[k]; de[n] = ex[k]; ++n; }
    for (int i = 1; i < n; ++i)   // insertion sort by stride
        for (int j = i; j > 0 && ds[j] < ds[j - 1]; --j) {
            const int64_t a = ds[j], e = de[j];
            ds[j] = ds[j - 1]; de[j] = de[j - 1];
            ds[j - 1] = a; de[j - 1] = e;
        }
    int64_t need = 1;
    for (int i = 0; i < n; ++i) {
        if (ds[i] < need) return false;
        if (!mul_ok(ds[i], de[i], &need)) return false;
    }
    return true;
}

int check_dtype_d(int dtype, int d) {
    if (dtype == DIFFATTN_BF16) return d == 64 ? DIFFATTN_OK : DIFFATTN_ERR_UNSUPPORTED;
    if (dtype == DIFFATTN_F32) return (d == 8 || d == 64) ? DIFFATTN_OK : DIFFATTN_ERR_UNSUPPORTED;
    return DIFFATTN_ERR_UNSUPPORTED;
}

size_t elem_bytes(int dtype) { return dtype == DIFFATTN_BF16 ? 2 : 4; }

int make_epilogue(float lambda, int layer, Epilogue* ep) {
    if (layer < 0) return DIFFATTN_ERR_LAYER;
    if (!isfinite(lambda)) return DIFFATTN_ERR_LAMBDA;
    ep->lambda = lambda;
    ep->normalise = layer >= 1 ? 1 : 0;
    ep->out_scale = layer >= 1 ? (float)(1.0 - diffattn_lambda_init(layer)) : 1.0f;
    ep->lambda_heads = nullptr;
    ep->heads = 1;
    return DIFFATTN_OK;
}

// Per-head lambda: a device array of H floats, 4-byte aligned, that the call must not write.
int check_lambda_heads(const float* lambda_heads, int64_t H, Span out) {
    if (!lambda_heads) return DIFFATTN_ERR_NULL;
    if (((uintptr_t)lambda_heads & 3u) != 0) return DIFFATTN_ERR_ALIGN;
    const Span l{(uintptr_t)lambda_heads, (uintptr_t)lambda_heads + (size_t)H * sizeof(float)};
    if (overlaps(l, out)) return DIFFATTN_ERR_ALIAS;
    return DIFFATTN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_ERR_HIP; }

}  // namespace

extern "C" {

double diffattn_lambda_init(int layer) {
    if (layer < 1) return NAN;
    return 0.8 - 0.6 * exp(-0.3 * (double)(layer - 1));
}

const char* diffattn_status_str(int status) {
    switch (status) {
        case DIFFATTN_OK: return "ok";
        case DIFFATTN_ERR_NULL: return "a required pointer is NULL";
        case DIFFATTN_ERR_SHAPE: return "invalid or unsupported size";
        case DIFFATTN_ERR_UNSUPPORTED: return "unsupported dtype / head width combination";
        case DIFFATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
        case DIFFATTN_ERR_LAYER: return "layer index must be >= 0";
        case DIFFATTN_ERR_LAMBDA: return "lambda must be finite";
        case DIFFATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case DIFFATTN_ERR_ALIAS: return "output or workspace overlaps another argument";
        case DIFFATTN_ERR_HIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

int diffattn_abi_version(void) { return ABI_VERSION; }

}  // extern "C"

namespace {

int fwd_impl(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out, int64_t B,
             int64_t H, int64_t N, int d, int dtype, float lambda, const float* lambda_heads, bool per_head, int layer,
             int causal, void* stream) {
    if (B < 0 || H < 0 || N < 0) return DIFFATTN_ERR_SHAPE;
    int st = check_dtype_d(dtype, d);
    if (st) return st;
    Epilogue ep;
    st = make_epilogue(per_head ? 0.0f : lambda, layer, &ep);
    if (st) return st;
    if (N > DIFFATTN_MAX_LEN) return DIFFATTN_ERR_SHAPE;
    int64_t BH, rows, qk_elems, v_elems;
    if (!mul_ok(B, H, &BH) || BH > INT32_MAX || !mul_ok(BH, N, &rows) || !mul_ok(rows, d, &qk_elems) ||
        !mul_ok(rows, 2 * (int64_t)d, &v_elems))
        return DIFFATTN_ERR_SHAPE;
    if (rows == 0) return DIFFATTN_OK;
    if (!q1 || !k1 || !q2 || !k2 || !v || !out) return DIFFATTN_ERR_NULL;
    if (!aligned16(q1) || !aligned16(k1) || !aligned16(q2) || !aligned16(k2) || !aligned16(v) || !aligned16(out))
        return DIFFATTN_ERR_ALIGN;
    const size_t eb = elem_bytes(dtype);
    const size_t qk_bytes = (size_t)qk_elems * eb, v_bytes = (size_t)v_elems * eb;
    const Span o{(uintptr_t)out, (uintptr_t)out + v_bytes};
    const Span ins[5] = {{(uintptr_t)q1, (uintptr_t)q1 + qk_bytes}, {(uintptr_t)k1, (uintptr_t)k1 + qk_bytes},
                         {(uintptr_t)q2, (uintptr_t)q2 + qk_bytes}, {(uintptr_t)k2, (uintptr_t)k2 + qk_bytes},
                         {(uintptr_t)v, (uintptr_t)v + v_bytes}};
    for (const Span& s : ins)
        if (overlaps(o, s)) return DIFFATTN_ERR_ALIAS;
    if (per_head) {
        st = check_lambda_heads(lambda_heads, H, o);
        if (st) return st;
        ep.lambda_heads = lambda_heads;
        ep.heads = (int)H;
    }

    hipStream_t s = (hipStream_t)stream;
    if (dtype == DIFFATTN_BF16)
        return hip_status(diffattn::launch_prefill_bf16_d64((const uint16_t*)q1, (const uint16_t*)k1,
                                                            (const uint16_t*)q2, (const uint16_t*)k2,
                                                            (const uint16_t*)v, (uint16_t*)out, B, H, N, causal,
                                                            diffattn::contiguous_strides(H, N, d), ep, nullptr, s));
    return hip_status(diffattn::launch_attn_f32((const float*)q1, (const float*)k1, (const float*)q2, (const float*)k2,
                                                (const float*)v, (float*)out, BH, N, N, d, causal, ep, s));
}

}  // namespace

extern "C" {

int diffattn_fwd(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out, int64_t B,
                 int64_t H, int64_t N, int d, int dtype, float lambda, int layer, int causal, void* stream) {
    return fwd_impl(q1, k1, q2, k2, v, out, B, H, N, d, dtype, lambda, nullptr, false, layer, causal, stream);
}

int diffattn_fwd_heads(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out,
                       int64_t B, int64_t H, int64_t N, int d, int dtype, const float* lambda_heads, int layer,
                       int causal, void* stream) {
    return fwd_impl(q1, k1, q2, k2, v, out, B, H, N, d, dtype, 0.0f, lambda_heads, true, layer, causal, stream);
}

int diffattn_fwd_strided(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out,
                         int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda, const float* lambda_heads,
                         int layer, int causal, const int64_t* strides, void* stream) {
    if (B < 0 || H < 0 || N < 0 || N > DIFFATTN_MAX_LEN) return DIFFATTN_ERR_SHAPE;
    if (dtype != DIFFATTN_BF16 || d != 64) return DIFFATTN_ERR_UNSUPPORTED;
    Epilogue ep;
    int st = make_epilogue(lambda_heads ? 0.0f : lambda, layer, &ep);
    if (st) return st;
    int64_t BH;
    if (!mul_ok(B, H, &BH) || BH > INT32_MAX) return DIFFATTN_ERR_SHAPE;
    if (BH == 0 || N == 0) return DIFFATTN_OK;
    if (!strides) return DIFFATTN_ERR_NULL;
    if (!q1 || !k1 || !q2 || !k2 || !v || !out) return DIFFATTN_ERR_NULL;
    if (!aligned16(q1) || !aligned16(k1) || !aligned16(q2) || !aligned16(k2) || !aligned16(v) || !aligned16(out))
        return DIFFATTN_ERR_ALIGN;
    diffattn::Strides S;
    const void* ptr[6] = {q1, k1, q2, k2, v, out};
    Span span[6];
    for (int k = 0; k < 6; ++k) {
        S.b[k] = strides[3 * k];
        S.h[k] = strides[3 * k + 1];
        S.n[k] = strides[3 * k + 2];
        const int64_t w = (k == diffattn::S_V || k == diffattn::S_OUT) ? 128 : 64;
        if (S.b[k] < 0 || S.h[k] < 0 || S.n[k] < w) return DIFFATTN_ERR_SHAPE;
        // 16-byte aligned rows: every stride a multiple of 8 bf16 elements.
        if ((S.b[k] | S.h[k] | S.n[k]) & 7) return DIFFATTN_ERR_ALIGN;
        // Element offset of the last element, and the 32-bit range of one head's rows (plus the prefetch overrun
        // of the direct loads, 256 rows) for the tensors read through buffer offsets.
        int64_t last, t1, t2, t3;
        if (!mul_ok(B - 1, S.b[k], &t1) || !mul_ok(H - 1, S.h[k], &t2) || !mul_ok(N - 1, S.n[k], &t3) ||
            t1 > INT64_MAX / 4 || t2 > INT64_MAX / 4 || t3 > INT64_MAX / 4)
            return DIFFATTN_ERR_SHAPE;
        last = t1 + t2 + t3 + w;
        if (k == diffattn::S_K1 || k == diffattn::S_K2 || k == diffattn::S_V) {
            int64_t range;
            if (!mul_ok(N + 256, S.n[k] * 2, &range) || range + w * 2 > (int64_t)UINT32_MAX) return DIFFATTN_ERR_SHAPE;
        }
        span[k] = Span{(uintptr_t)ptr[k], (uintptr_t)ptr[k] + (uintptr_t)last * 2};
    }
    if (!one_to_one(B, H, N, 128, S.b[diffattn::S_OUT], S.h[diffattn::S_OUT], S.n[diffattn::S_OUT]))
        return DIFFATTN_ERR_ALIAS;
    for (int k = 0; k < 5; ++k)
        if (overlaps(span[diffattn::S_OUT], span[k])) return DIFFATTN_ERR_ALIAS;
    if (lambda_heads) {
        st = check_lambda_heads(lambda_heads, H, span[diffattn::S_OUT]);
        if (st) return st;
        ep.lambda_heads = lambda_heads;
        ep.heads = (int)H;
    }
    return hip_status(diffattn::launch_prefill_bf16_d64((const uint16_t*)q1, (const uint16_t*)k1, (const uint16_t*)q2,
                                                        (const uint16_t*)k2, (const uint16_t*)v, (uint16_t*)out, B, H,
                                                        N, causal, S, ep, nullptr, (hipStream_t)stream));
}

size_t diffattn_fwd_split_workspace_bytes(int64_t B, int64_t H, int64_t N, int d) {
    int64_t BH, rows, floats;
    if (B < 0 || H < 0 || N < 0 || N > DIFFATTN_MAX_LEN || d != 64 || !mul_ok(B, H, &BH) || BH > INT32_MAX ||
        !mul_ok(BH, N, &rows))
        return 0;
    const int splits = diffattn::prefill_key_splits_max(BH, N);
    if (splits <= 1 || !mul_ok(rows, (int64_t)splits * diffattn::PARTIAL_FLOATS, &floats) ||
        floats > INT64_MAX / 4)
        return 0;
    return (size_t)floats * sizeof(float);
}

int diffattn_fwd_split(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out,
                       int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda, const float* lambda_heads,
                       int layer, int causal, void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || H < 0 || N < 0 || N > DIFFATTN_MAX_LEN) return DIFFATTN_ERR_SHAPE;
    int st = check_dtype_d(dtype, d);
    if (st) return st;
    if (dtype != DIFFATTN_BF16 || d != 64) return DIFFATTN_ERR_UNSUPPORTED;
    Epilogue ep;
    st = make_epilogue(lambda_heads ? 0.0f : lambda, layer, &ep);
    if (st) return st;
    int64_t BH, rows, qk_elems, v_elems;
    if (!mul_ok(B, H, &BH) || BH > INT32_MAX || !mul_ok(BH, N, &rows) || rows > INT32_MAX ||
        !mul_ok(rows, d, &qk_elems) || !mul_ok(rows, 2 * (int64_t)d, &v_elems))
        return DIFFATTN_ERR_SHAPE;
    if (rows == 0) return DIFFATTN_OK;
    if (!q1 || !k1 || !q2 || !k2 || !v || !out) return DIFFATTN_ERR_NULL;
    if (!aligned16(q1) || !aligned16(k1) || !aligned16(q2) || !aligned16(k2) || !aligned16(v) || !aligned16(out))
        return DIFFATTN_ERR_ALIGN;
    const size_t qk_bytes = (size_t)qk_elems * 2, v_bytes = (size_t)v_elems * 2;
    const Span o{(uintptr_t)out, (uintptr_t)out + v_bytes};
    const Span ins[5] = {{(uintptr_t)q1, (uintptr_t)q1 + qk_bytes}, {(uintptr_t)k1, (uintptr_t)k1 + qk_bytes},
                         {(uintptr_t)q2, (uintptr_t)q2 + qk_bytes}, {(uintptr_t)k2, (uintptr_t)k2 + qk_bytes},
                         {(uintptr_t)v, (uintptr_t)v + v_bytes}};
    for (const Span& s : ins)
        if (overlaps(o, s)) return DIFFATTN_ERR_ALIAS;
    if (lambda_heads) {
        st = check_lambda_heads(lambda_heads, H, o);
        if (st) return st;
        ep.lambda_heads = lambda_heads;
        ep.heads = (int)H;
    }
    const size_t need = diffattn_fwd_split_workspace_bytes(B, H, N, d);
    if (need > 0) {
        if (!workspace) return DIFFATTN_ERR_WORKSPACE;
        if (!aligned16(workspace)) return DIFFATTN_ERR_ALIGN;
        if (workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
        const Span w{(uintptr_t)workspace, (uintptr_t)workspace + need};
        if (overlaps(w, o)) return DIFFATTN_ERR_ALIAS;
        for (const Span& s : ins)
            if (overlaps(w, s)) return DIFFATTN_ERR_ALIAS;
        if (lambda_heads &&
            overlaps(w, Span{(uintptr_t)lambda_heads, (uintptr_t)lambda_heads + (size_t)H * sizeof(float)}))
            return DIFFATTN_ERR_ALIAS;
    }
    return hip_status(diffattn::launch_prefill_split_bf16_d64(
        (const uint16_t*)q1, (const uint16_t*)k1, (const uint16_t*)q2, (const uint16_t*)k2, (const uint16_t*)v,
        (uint16_t*)out, B, H, N, causal, ep, (float*)workspace, (hipStream_t)stream));
}

size_t diffattn_decode_workspace_bytes(int64_t B, int64_t H, int64_t L, int d) {
    int64_t BH;
    if (B < 0 || H < 0 || L <= 0 || L > DIFFATTN_MAX_LEN || d != 64 || !mul_ok(B, H, &BH) || BH > INT32_MAX)
        return 0;
    return diffattn::decode_bf16_workspace_bytes(BH, H, L, 1, false);
}

size_t diffattn_decode_varlen_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t L, int d) {
    int64_t BH;
    if (B < 0 || H < 0 || T < 1 || T > DIFFATTN_MAX_NEW_TOKENS || L < T || L > DIFFATTN_MAX_LEN || d != 64 ||
        !mul_ok(B, H, &BH) || BH > INT32_MAX)
        return 0;
    return diffattn::decode_bf16_workspace_bytes(BH, H, L, (int)T, true);
}

}  // extern "C"

namespace {

// strided: the caches are addressed through cache_strides, 9 host values (k1, k2, v: batch, head, row; elements);
// otherwise they are dense [B][H][L][w].
int decode_impl(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out, int64_t B,
                int64_t H, int64_t T, int64_t L, const int32_t* lens, bool varlen, int d, int dtype, float lambda,
                const float* lambda_heads, bool per_head, int layer, void* workspace, size_t workspace_bytes,
                void* stream, bool strided = false, const int64_t* cache_strides = nullptr) {
    if (B < 0 || H < 0 || L < 0 || T < 1) return DIFFATTN_ERR_SHAPE;
    if (L == 0 || L > DIFFATTN_MAX_LEN || T > DIFFATTN_MAX_NEW_TOKENS || L < T) return DIFFATTN_ERR_SHAPE;
    int st = check_dtype_d(dtype, d);
    if (st) return st;
    if (varlen && dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
    Epilogue ep;
    st = make_epilogue(per_head ? 0.0f : lambda, layer, &ep);
    if (st) return st;
    int64_t BH, q_rows, q_elems, kv_rows, k_elems, v_elems;
    if (!mul_ok(B, H, &BH) || BH > INT32_MAX || !mul_ok(BH, T, &q_rows) || !mul_ok(q_rows, d, &q_elems) ||
        !mul_ok(BH, L, &kv_rows) || !mul_ok(kv_rows, d, &k_elems) || !mul_ok(kv_rows, 2 * (int64_t)d, &v_elems))
        return DIFFATTN_ERR_SHAPE;
    if (BH == 0) return DIFFATTN_OK;
    if (!q1 || !k1 || !q2 || !k2 || !v || !out) return DIFFATTN_ERR_NULL;
    if (strided && !cache_strides) return DIFFATTN_ERR_NULL;
    if (!aligned16(q1) || !aligned16(k1) || !aligned16(q2) || !aligned16(k2) || !aligned16(v) || !aligned16(out))
        return DIFFATTN_ERR_ALIGN;
    const size_t eb = elem_bytes(dtype);
    diffattn::CacheStrides cs = diffattn::dense_cache_strides(H, L, d);
    Span cache_span[3] = {{(uintptr_t)k1, (uintptr_t)k1 + (size_t)k_elems * eb},
                          {(uintptr_t)k2, (uintptr_t)k2 + (size_t)k_elems * eb},
                          {(uintptr_t)v, (uintptr_t)v + (size_t)v_elems * eb}};
    if (strided) {
        if (dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
        const void* cp[3] = {k1, k2, v};
        for (int k = 0; k < 3; ++k) {
            cs.b[k] = cache_strides[3 * k];
            cs.h[k] = cache_strides[3 * k + 1];
            cs.n[k] = cache_strides[3 * k + 2];
            const int64_t w = k == diffattn::C_V ? 2 * (int64_t)d : d;
            if (cs.b[k] < 0 || cs.h[k] < 0 || cs.n[k] < w) return DIFFATTN_ERR_SHAPE;
            if ((cs.b[k] | cs.h[k] | cs.n[k]) & 7) return DIFFATTN_ERR_ALIGN;   // 16-byte aligned rows
            int64_t t1, t2, t3;
            if (!mul_ok(B - 1, cs.b[k], &t1) || !mul_ok(H - 1, cs.h[k], &t2) || !mul_ok(L - 1, cs.n[k], &t3) ||
                t1 > INT64_MAX / 4 || t2 > INT64_MAX / 4 || t3 > INT64_MAX / 4)
                return DIFFATTN_ERR_SHAPE;
            cache_span[k] = Span{(uintptr_t)cp[k], (uintptr_t)cp[k] + (uintptr_t)(t1 + t2 + t3 + w) * eb};
        }
    }
    const Span o{(uintptr_t)out, (uintptr_t)out + (size_t)q_elems * 2 * eb};
    const Span ins[5] = {{(uintptr_t)q1, (uintptr_t)q1 + (size_t)q_elems * eb}, cache_span[0],
                         {(uintptr_t)q2, (uintptr_t)q2 + (size_t)q_elems * eb}, cache_span[1], cache_span[2]};
    for (const Span& s : ins)
        if (overlaps(o, s)) return DIFFATTN_ERR_ALIAS;
    if (per_head) {
        st = check_lambda_heads(lambda_heads, H, o);
        if (st) return st;
        ep.lambda_heads = lambda_heads;
        ep.heads = (int)H;
    }
    const Span ls{(uintptr_t)lens, (uintptr_t)lens + (size_t)B * sizeof(int32_t)};
    if (lens) {
        if (((uintptr_t)lens & 3u) != 0) return DIFFATTN_ERR_ALIGN;
        if (overlaps(ls, o)) return DIFFATTN_ERR_ALIAS;
    }

    hipStream_t s = (hipStream_t)stream;
    if (dtype == DIFFATTN_F32)  // exact fp32 path: one query row per head at the end of the cache
        return hip_status(diffattn::launch_attn_f32((const float*)q1, (const float*)k1, (const float*)q2,
                                                    (const float*)k2, (const float*)v, (float*)out, BH, 1, L, d, 1, ep,
                                                    s));

    const size_t need = diffattn::decode_bf16_workspace_bytes(BH, H, L, (int)T, lens != nullptr);
    if (!workspace || workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DIFFATTN_ERR_ALIGN;
    const Span w{(uintptr_t)workspace, (uintptr_t)workspace + need};
    if (overlaps(w, o)) return DIFFATTN_ERR_ALIAS;
    for (const Span& sp : ins)
        if (overlaps(w, sp)) return DIFFATTN_ERR_ALIAS;
    if (per_head && overlaps(w, Span{(uintptr_t)lambda_heads, (uintptr_t)lambda_heads + (size_t)H * sizeof(float)}))
        return DIFFATTN_ERR_ALIAS;
    if (lens && overlaps(w, ls)) return DIFFATTN_ERR_ALIAS;
    return hip_status(diffattn::launch_decode_bf16_d64((const uint16_t*)q1, (const uint16_t*)k1, (const uint16_t*)q2,
                                                       (const uint16_t*)k2, (const uint16_t*)v, (uint16_t*)out, BH, H,
                                                       L, (int)T, lens, nullptr, cs, ep, workspace, s));
}

}  // namespace

extern "C" {

// Scratch of the allocation-free decode: one array per GPU, held from the library's load until the process ends.
// In host code `scratch` is a host-side stand-in, not a device address: the device address of each GPU's copy is
// looked up once per device, with that device current, and only that address is ever passed to a kernel.
namespace {
__device__ __attribute__((aligned(256))) unsigned char scratch[DIFFATTN_NOALLOC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::once_flag scratch_once[MAX_DEVICES];
void* scratch_ptr[MAX_DEVICES];
hipError_t scratch_err[MAX_DEVICES];

// Device address of the current device's scratch array (DIFFATTN_ERR_HIP if it cannot be found).
int scratch_of_current_device(void** p) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return DIFFATTN_ERR_HIP;
    std::call_once(scratch_once[dev], [dev] {
        scratch_err[dev] = hipGetSymbolAddress(&scratch_ptr[dev], HIP_SYMBOL(scratch));
    });
    if (scratch_err[dev] != hipSuccess || !scratch_ptr[dev]) return DIFFATTN_ERR_HIP;
    *p = scratch_ptr[dev];
    return DIFFATTN_OK;
}
}  // namespace

int diffattn_decode_noalloc(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out,
                            int64_t B, int64_t H, int64_t L, int d, int dtype, float lambda, int layer, int causal,
                            void* stream) {
    (void)causal;
    // Size check first, before any HIP call; invalid shapes (need 0) are reported by decode_impl.
    const size_t need = dtype == DIFFATTN_BF16 ? diffattn_decode_workspace_bytes(B, H, L, d) : 0;
    if (need > DIFFATTN_NOALLOC_SCRATCH_BYTES) return DIFFATTN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const int st = scratch_of_current_device(&ws);
        if (st) return st;
    }
    return decode_impl(q1, k1, q2, k2, v, out, B, H, 1, L, nullptr, false, d, dtype, lambda, nullptr, false, layer, ws,
                       ws ? (size_t)DIFFATTN_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int diffattn_decode(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out,
                    int64_t B, int64_t H, int64_t L, int d, int dtype, float lambda, int layer, int causal,
                    void* workspace, size_t workspace_bytes, void* stream) {
    (void)causal;  // the single query is the last position: every cached key is visible either way
    return decode_impl(q1, k1, q2, k2, v, out, B, H, 1, L, nullptr, false, d, dtype, lambda, nullptr, false, layer,
                       workspace, workspace_bytes, stream);
}

int diffattn_decode_heads(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out,
                          int64_t B, int64_t H, int64_t L, int d, int dtype, const float* lambda_heads, int layer,
                          int causal, void* workspace, size_t workspace_bytes, void* stream) {
    (void)causal;
    return decode_impl(q1, k1, q2, k2, v, out, B, H, 1, L, nullptr, false, d, dtype, 0.0f, lambda_heads, true, layer,
                       workspace, workspace_bytes, stream);
}

namespace {

// Page size checks of the paged decode: a power of two in [16, DIFFATTN_MAX_PAGE_SIZE]; returns log2, or -1.
int page_log2(int64_t page_size) {
    if (page_size < 16 || page_size > DIFFATTN_MAX_PAGE_SIZE || (page_size & (page_size - 1)) != 0) return -1;
    int l = 0;
    while ((int64_t{1} << l) < page_size) ++l;
    return l;
}

}  // namespace

size_t diffattn_decode_paged_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t max_pages, int64_t page_size,
                                             int d) {
    int64_t L;
    if (max_pages < 1 || page_log2(page_size) < 0 || !mul_ok(max_pages, page_size, &L)) return 0;
    return diffattn_decode_varlen_workspace_bytes(B, H, T, L, d);
}

int diffattn_decode_paged(const void* q1, const void* k1_pages, const void* q2, const void* k2_pages,
                          const void* v_pages, void* out, int64_t B, int64_t H, int64_t T,
                          const int32_t* block_table, int64_t max_pages, int64_t page_size, int64_t num_pages,
                          const int32_t* lens, int d, int dtype, float lambda, const float* lambda_heads, int layer,
                          void* workspace, size_t workspace_bytes, void* stream) {
    const int lp = page_log2(page_size);
    int64_t L;
    if (B < 0 || H < 0 || T < 1 || T > DIFFATTN_MAX_NEW_TOKENS || max_pages < 1 || max_pages > INT32_MAX ||
        num_pages < 1 || num_pages > INT32_MAX || lp < 0 || !mul_ok(max_pages, page_size, &L) ||
        L > DIFFATTN_MAX_LEN || L < T)
        return DIFFATTN_ERR_SHAPE;
    int st = check_dtype_d(dtype, d);
    if (st) return st;
    if (dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
    Epilogue ep;
    st = make_epilogue(lambda_heads ? 0.0f : lambda, layer, &ep);
    if (st) return st;
    int64_t BH, q_elems, pool_rows, k_elems, v_elems, table_elems;
    if (!mul_ok(B, H, &BH) || BH > INT32_MAX || !mul_ok(BH * T, d, &q_elems) || !mul_ok(num_pages, H, &pool_rows) ||
        !mul_ok(pool_rows, page_size, &pool_rows) || !mul_ok(pool_rows, d, &k_elems) ||
        !mul_ok(pool_rows, 2 * (int64_t)d, &v_elems) || !mul_ok(B, max_pages, &table_elems))
        return DIFFATTN_ERR_SHAPE;
    if (BH == 0) return DIFFATTN_OK;
    if (!q1 || !k1_pages || !q2 || !k2_pages || !v_pages || !out || !block_table) return DIFFATTN_ERR_NULL;
    if (!aligned16(q1) || !aligned16(k1_pages) || !aligned16(q2) || !aligned16(k2_pages) || !aligned16(v_pages) ||
        !aligned16(out) || ((uintptr_t)block_table & 3u) != 0 || ((uintptr_t)lens & 3u) != 0)
        return DIFFATTN_ERR_ALIGN;
    const Span o{(uintptr_t)out, (uintptr_t)out + (size_t)q_elems * 2 * 2};
    const Span ins[7] = {{(uintptr_t)q1, (uintptr_t)q1 + (size_t)q_elems * 2},
                         {(uintptr_t)k1_pages, (uintptr_t)k1_pages + (size_t)k_elems * 2},
                         {(uintptr_t)q2, (uintptr_t)q2 + (size_t)q_elems * 2},
                         {(uintptr_t)k2_pages, (uintptr_t)k2_pages + (size_t)k_elems * 2},
                         {(uintptr_t)v_pages, (uintptr_t)v_pages + (size_t)v_elems * 2},
                         {(uintptr_t)block_table, (uintptr_t)block_table + (size_t)table_elems * 4},
                         {(uintptr_t)lens, (uintptr_t)lens + (lens ? (size_t)B * 4 : 0)}};
    for (const Span& sp : ins)
        if (overlaps(o, sp)) return DIFFATTN_ERR_ALIAS;
    if (lambda_heads) {
        st = check_lambda_heads(lambda_heads, H, o);
        if (st) return st;
        ep.lambda_heads = lambda_heads;
        ep.heads = (int)H;
    }
    const size_t need = diffattn::decode_bf16_workspace_bytes(BH, H, L, (int)T, lens != nullptr);
    if (!workspace || workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DIFFATTN_ERR_ALIGN;
    const Span w{(uintptr_t)workspace, (uintptr_t)workspace + need};
    if (overlaps(w, o)) return DIFFATTN_ERR_ALIAS;
    for (const Span& sp : ins)
        if (overlaps(w, sp)) return DIFFATTN_ERR_ALIAS;
    if (lambda_heads && overlaps(w, Span{(uintptr_t)lambda_heads, (uintptr_t)lambda_heads + (size_t)H * sizeof(float)}))
        return DIFFATTN_ERR_ALIAS;
    const diffattn::DecodePages pg{block_table, (int)max_pages, lp, (int)num_pages};
    return hip_status(diffattn::launch_decode_bf16_d64(
        (const uint16_t*)q1, (const uint16_t*)k1_pages, (const uint16_t*)q2, (const uint16_t*)k2_pages,
        (const uint16_t*)v_pages, (uint16_t*)out, BH, H, L, (int)T, lens, &pg, diffattn::dense_cache_strides(H, L, d), ep,
        workspace, (hipStream_t)stream));
}

int diffattn_decode_varlen(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out,
                           int64_t B, int64_t H, int64_t T, int64_t L, const int32_t* lens, int d, int dtype,
                           float lambda, const float* lambda_heads, int layer, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return decode_impl(q1, k1, q2, k2, v, out, B, H, T, L, lens, true, d, dtype, lambda_heads ? 0.0f : lambda,
                       lambda_heads, lambda_heads != nullptr, layer, workspace, workspace_bytes, stream);
}

int diffattn_decode_strided(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out,
                            int64_t B, int64_t H, int64_t T, int64_t L, const int32_t* lens,
                            const int64_t* cache_strides, int d, int dtype, float lambda, const float* lambda_heads,
                            int layer, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(q1, k1, q2, k2, v, out, B, H, T, L, lens, true, d, dtype, lambda_heads ? 0.0f : lambda,
                       lambda_heads, lambda_heads != nullptr, layer, workspace, workspace_bytes, stream, true,
                       cache_strides);
}


size_t diffattn_train_saved_bytes(int64_t B, int64_t H, int64_t N, int d) {
    int64_t BH, rows;
    if (B < 0 || H < 0 || N < 0 || N > DIFFATTN_MAX_LEN || d != 64 || !mul_ok(B, H, &BH) || BH > INT32_MAX ||
        !mul_ok(BH, N, &rows))
        return 0;
    return (size_t)rows * diffattn::SAVED_FLOATS * sizeof(float);
}

size_t diffattn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int d) {
    int64_t BH, rows;
    if (B < 0 || H < 0 || N < 0 || N > DIFFATTN_MAX_LEN || d != 64 || !mul_ok(B, H, &BH) || BH > INT32_MAX ||
        !mul_ok(BH, N, &rows) || rows == 0)
        return 0;
    return diffattn::bwd_bf16_workspace_bytes(BH, N);
}

int diffattn_fwd_train(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, void* out,
                       int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda, const float* lambda_heads,
                       int layer, int causal, void* saved, size_t saved_bytes, void* stream) {
    if (B < 0 || H < 0 || N < 0 || N > DIFFATTN_MAX_LEN) return DIFFATTN_ERR_SHAPE;
    if (dtype != DIFFATTN_BF16 || d != 64) return DIFFATTN_ERR_UNSUPPORTED;
    Epilogue ep;
    int st = make_epilogue(lambda_heads ? 0.0f : lambda, layer, &ep);
    if (st) return st;
    int64_t BH, rows;
    if (!mul_ok(B, H, &BH) || BH > INT32_MAX || !mul_ok(BH, N, &rows)) return DIFFATTN_ERR_SHAPE;
    if (rows == 0) return DIFFATTN_OK;
    if (!q1 || !k1 || !q2 || !k2 || !v || !out || !saved) return DIFFATTN_ERR_NULL;
    if (!aligned16(q1) || !aligned16(k1) || !aligned16(q2) || !aligned16(k2) || !aligned16(v) || !aligned16(out) ||
        !aligned16(saved))
        return DIFFATTN_ERR_ALIGN;
    const size_t need = diffattn_train_saved_bytes(B, H, N, d);
    if (saved_bytes < need) return DIFFATTN_ERR_WORKSPACE;
    const size_t qk = (size_t)rows * 64 * 2, vb = (size_t)rows * 128 * 2;
    const Span ins[5] = {{(uintptr_t)q1, (uintptr_t)q1 + qk}, {(uintptr_t)k1, (uintptr_t)k1 + qk},
                         {(uintptr_t)q2, (uintptr_t)q2 + qk}, {(uintptr_t)k2, (uintptr_t)k2 + qk},
                         {(uintptr_t)v, (uintptr_t)v + vb}};
    const Span o{(uintptr_t)out, (uintptr_t)out + vb}, sv{(uintptr_t)saved, (uintptr_t)saved + need};
    if (overlaps(o, sv)) return DIFFATTN_ERR_ALIAS;
    for (const Span& sp : ins)
        if (overlaps(o, sp) || overlaps(sv, sp)) return DIFFATTN_ERR_ALIAS;
    if (lambda_heads) {
        st = check_lambda_heads(lambda_heads, H, o);
        if (st) return st;
        if (overlaps(sv, Span{(uintptr_t)lambda_heads, (uintptr_t)lambda_heads + (size_t)H * sizeof(float)}))
            return DIFFATTN_ERR_ALIAS;
        ep.lambda_heads = lambda_heads;
        ep.heads = (int)H;
    }
    return hip_status(diffattn::launch_prefill_bf16_d64((const uint16_t*)q1, (const uint16_t*)k1, (const uint16_t*)q2,
                                                        (const uint16_t*)k2, (const uint16_t*)v, (uint16_t*)out, B, H,
                                                        N, causal, diffattn::contiguous_strides(H, N, d), ep,
                                                        (float*)saved, (hipStream_t)stream));
}

int diffattn_bwd(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, const void* dy,
                 const void* saved, void* dq1, void* dk1, void* dq2, void* dk2, void* dv, float* dlambda, int64_t B,
                 int64_t H, int64_t N, int d, int dtype, float lambda, const float* lambda_heads, int layer,
                 int causal, void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || H < 0 || N < 0 || N > DIFFATTN_MAX_LEN) return DIFFATTN_ERR_SHAPE;
    if (dtype != DIFFATTN_BF16 || d != 64) return DIFFATTN_ERR_UNSUPPORTED;
    Epilogue ep;
    int st = make_epilogue(lambda_heads ? 0.0f : lambda, layer, &ep);
    if (st) return st;
    int64_t BH, rows;
    if (!mul_ok(B, H, &BH) || BH > INT32_MAX || !mul_ok(BH, N, &rows)) return DIFFATTN_ERR_SHAPE;
    if (BH == 0) return DIFFATTN_OK;
    if (!dlambda) return DIFFATTN_ERR_NULL;
    if (((uintptr_t)dlambda & 3u) != 0) return DIFFATTN_ERR_ALIGN;
    if (rows == 0)   // no rows: dlambda is zero (written by a kernel, so the call stays capturable in a graph)
        return hip_status(diffattn::launch_bwd_bf16_d64(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                         nullptr, nullptr, nullptr, nullptr, nullptr, dlambda, B, H, 0,
                                                         causal, ep, diffattn::dense_bwd_strides(H, 0, d), nullptr,
                                                         (hipStream_t)stream));
    if (!q1 || !k1 || !q2 || !k2 || !v || !dy || !saved || !dq1 || !dk1 || !dq2 || !dk2 || !dv) return DIFFATTN_ERR_NULL;
    const void* a16[] = {q1, k1, q2, k2, v, dy, saved, dq1, dk1, dq2, dk2, dv};
    for (const void* p : a16)
        if (!aligned16(p)) return DIFFATTN_ERR_ALIGN;
    const size_t need = diffattn_bwd_workspace_bytes(B, H, N, d);
    if (!workspace || workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return DIFFATTN_ERR_ALIGN;
    const size_t qk = (size_t)rows * 64 * 2, vb = (size_t)rows * 128 * 2;
    const size_t sb = diffattn_train_saved_bytes(B, H, N, d);
    const Span ins[7] = {{(uintptr_t)q1, (uintptr_t)q1 + qk}, {(uintptr_t)k1, (uintptr_t)k1 + qk},
                         {(uintptr_t)q2, (uintptr_t)q2 + qk}, {(uintptr_t)k2, (uintptr_t)k2 + qk},
                         {(uintptr_t)v, (uintptr_t)v + vb}, {(uintptr_t)dy, (uintptr_t)dy + vb},
                         {(uintptr_t)saved, (uintptr_t)saved + sb}};
    const Span outs[7] = {{(uintptr_t)dq1, (uintptr_t)dq1 + qk}, {(uintptr_t)dk1, (uintptr_t)dk1 + qk},
                          {(uintptr_t)dq2, (uintptr_t)dq2 + qk}, {(uintptr_t)dk2, (uintptr_t)dk2 + qk},
                          {(uintptr_t)dv, (uintptr_t)dv + vb},
                          {(uintptr_t)dlambda, (uintptr_t)dlambda + (size_t)H * sizeof(float)},
                          {(uintptr_t)workspace, (uintptr_t)workspace + need}};
    for (int i = 0; i < 7; ++i) {
        for (const Span& sp : ins)
            if (overlaps(outs[i], sp)) return DIFFATTN_ERR_ALIAS;
        for (int j = i + 1; j < 7; ++j)
            if (overlaps(outs[i], outs[j])) return DIFFATTN_ERR_ALIAS;
    }
    if (lambda_heads) {
        if (((uintptr_t)lambda_heads & 3u) != 0) return DIFFATTN_ERR_ALIGN;
        const Span l{(uintptr_t)lambda_heads, (uintptr_t)lambda_heads + (size_t)H * sizeof(float)};
        for (const Span& sp : outs)
            if (overlaps(l, sp)) return DIFFATTN_ERR_ALIAS;
        ep.lambda_heads = lambda_heads;
        ep.heads = (int)H;
    }
    return hip_status(diffattn::launch_bwd_bf16_d64(
        (const uint16_t*)q1, (const uint16_t*)k1, (const uint16_t*)q2, (const uint16_t*)k2, (const uint16_t*)v,
        (const uint16_t*)dy, (const float*)saved, (uint16_t*)dq1, (uint16_t*)dk1, (uint16_t*)dq2, (uint16_t*)dk2,
        (uint16_t*)dv, dlambda, B, H, N, causal, ep, diffattn::dense_bwd_strides(H, N, d), workspace,
        (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Byte footprint of one strided bf16 tensor [B][H][N][w] for overlap checks: its bounding box, the byte strides of
// its dimensions of extent > 1 (0 for the others) and its row width in bytes.
struct Footprint {
    uintptr_t lo, hi;
    int64_t sb, sh, sn, wb;
};

Footprint dense_footprint(const void* p, size_t bytes) {
    return Footprint{(uintptr_t)p, (uintptr_t)p + bytes, 0, 0, 0, (int64_t)bytes};
}

// Validates one strided tensor (element strides s[0..2] for batch, head and row; rows of w contiguous elements) and
// returns its footprint.  `buffered` tensors are read through 32-bit buffer offsets: one head's N + 256 rows must
// span less than 4 GiB.
int strided_tensor(const void* p, int64_t B, int64_t H, int64_t N, int64_t w, const int64_t* s, bool buffered,
                   Footprint* f) {
    const int64_t sb = s[0], sh = s[1], sn = s[2];
    if (sb < 0 || sh < 0 || sn < w) return DIFFATTN_ERR_SHAPE;
    if ((sb | sh | sn) & 7) return DIFFATTN_ERR_ALIGN;   // 16-byte aligned rows
    int64_t t1, t2, t3;
    if (!mul_ok(B - 1, sb, &t1) || !mul_ok(H - 1, sh, &t2) || !mul_ok(N - 1, sn, &t3) || t1 > INT64_MAX / 4 ||
        t2 > INT64_MAX / 4 || t3 > INT64_MAX / 4)
        return DIFFATTN_ERR_SHAPE;
    if (buffered) {
        int64_t range;
        if (!mul_ok(N + 256, sn * 2, &range) || range + w * 2 > (int64_t)UINT32_MAX) return DIFFATTN_ERR_SHAPE;
    }
    *f = Footprint{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(t1 + t2 + t3 + w) * 2, B > 1 ? 2 * sb : 0,
                   H > 1 ? 2 * sh : 0, N > 1 ? 2 * sn : 0, 2 * w};
    return DIFFATTN_OK;
}

int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// True when two footprints provably share no byte: their bounding boxes are disjoint, or every byte of each lies at
// its base plus a multiple of m = gcd(all their strides) plus a column offset below its row width, and the two
// resulting arcs of residues modulo m do not meet (interleaved rows of one packed buffer).
bool disjoint(const Footprint& a, const Footprint& b) {
    if (!overlaps(Span{a.lo, a.hi}, Span{b.lo, b.hi})) return true;
    int64_t m = 0;
    for (int64_t x : {a.sb, a.sh, a.sn, b.sb, b.sh, b.sn}) m = gcd64(m, x);
    if (m == 0 || a.wb + b.wb > m) return false;
    const int64_t ra = (int64_t)(a.lo % (uint64_t)m), rb = (int64_t)(b.lo % (uint64_t)m);
    return ((rb - ra) % m + m) % m >= a.wb && ((ra - rb) % m + m) % m >= b.wb;
}

}  // namespace

extern "C" {

int diffattn_fwd_train_strided(const void* q1, const void* k1, const void* q2, const void* k2, const void* v,
                               void* out, int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda,
                               const float* lambda_heads, int layer, int causal, const int64_t* strides, void* saved,
                               size_t saved_bytes, void* stream) {
    if (B < 0 || H < 0 || N < 0 || N > DIFFATTN_MAX_LEN) return DIFFATTN_ERR_SHAPE;
    if (dtype != DIFFATTN_BF16 || d != 64) return DIFFATTN_ERR_UNSUPPORTED;
    Epilogue ep;
    int st = make_epilogue(lambda_heads ? 0.0f : lambda, layer, &ep);
    if (st) return st;
    int64_t BH, rows;
    if (!mul_ok(B, H, &BH) || BH > INT32_MAX || !mul_ok(BH, N, &rows)) return DIFFATTN_ERR_SHAPE;
    if (rows == 0) return DIFFATTN_OK;
    if (!strides || !q1 || !k1 || !q2 || !k2 || !v || !out || !saved) return DIFFATTN_ERR_NULL;
    const void* ptr[6] = {q1, k1, q2, k2, v, out};
    for (const void* p : ptr)
        if (!aligned16(p)) return DIFFATTN_ERR_ALIGN;
    if (!aligned16(saved)) return DIFFATTN_ERR_ALIGN;
    const size_t need = diffattn_train_saved_bytes(B, H, N, d);
    if (saved_bytes < need) return DIFFATTN_ERR_WORKSPACE;
    Footprint f[6];
    diffattn::Strides S;
    for (int k = 0; k < 6; ++k) {
        const bool wide = k == diffattn::S_V || k == diffattn::S_OUT;
        const bool buffered = k == diffattn::S_K1 || k == diffattn::S_K2 || k == diffattn::S_V;
        st = strided_tensor(ptr[k], B, H, N, wide ? 128 : 64, strides + 3 * k, buffered, &f[k]);
        if (st) return st;
        S.b[k] = strides[3 * k];
        S.h[k] = strides[3 * k + 1];
        S.n[k] = strides[3 * k + 2];
    }
    if (!one_to_one(B, H, N, 128, S.b[diffattn::S_OUT], S.h[diffattn::S_OUT], S.n[diffattn::S_OUT]))
        return DIFFATTN_ERR_ALIAS;
    const Footprint sv = dense_footprint(saved, need);
    if (!disjoint(f[diffattn::S_OUT], sv)) return DIFFATTN_ERR_ALIAS;
    for (int k = 0; k < 5; ++k)
        if (!disjoint(f[diffattn::S_OUT], f[k]) || !disjoint(sv, f[k])) return DIFFATTN_ERR_ALIAS;
    if (lambda_heads) {
        if (((uintptr_t)lambda_heads & 3u) != 0) return DIFFATTN_ERR_ALIGN;
        const Footprint l = dense_footprint(lambda_heads, (size_t)H * sizeof(float));
        if (!disjoint(l, f[diffattn::S_OUT]) || !disjoint(l, sv)) return DIFFATTN_ERR_ALIAS;
        ep.lambda_heads = lambda_heads;
        ep.heads = (int)H;
    }
    return hip_status(diffattn::launch_prefill_bf16_d64((const uint16_t*)q1, (const uint16_t*)k1, (const uint16_t*)q2,
                                                        (const uint16_t*)k2, (const uint16_t*)v, (uint16_t*)out, B, H,
                                                        N, causal, S, ep, (float*)saved, (hipStream_t)stream));
}

int diffattn_bwd_strided(const void* q1, const void* k1, const void* q2, const void* k2, const void* v,
                         const void* dy, const void* saved, void* dq1, void* dk1, void* dq2, void* dk2, void* dv,
                         float* dlambda, int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda,
                         const float* lambda_heads, int layer, int causal, const int64_t* strides, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (B < 0 || H < 0 || N < 0 || N > DIFFATTN_MAX_LEN) return DIFFATTN_ERR_SHAPE;
    if (dtype != DIFFATTN_BF16 || d != 64) return DIFFATTN_ERR_UNSUPPORTED;
    Epilogue ep;
    int st = make_epilogue(lambda_heads ? 0.0f : lambda, layer, &ep);
    if (st) return st;
    int64_t BH, rows;
    if (!mul_ok(B, H, &BH) || BH > INT32_MAX || !mul_ok(BH, N, &rows)) return DIFFATTN_ERR_SHAPE;
    if (BH == 0) return DIFFATTN_OK;
    if (!dlambda) return DIFFATTN_ERR_NULL;
    if (((uintptr_t)dlambda & 3u) != 0) return DIFFATTN_ERR_ALIGN;
    if (rows == 0)   // no rows: dlambda is zero, as for diffattn_bwd
        return diffattn_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, dlambda, B, H, N, d, dtype, lambda, lambda_heads, layer, causal, nullptr,
                            0, stream);
    if (!strides || !q1 || !k1 || !q2 || !k2 || !v || !dy || !saved || !dq1 || !dk1 || !dq2 || !dk2 || !dv)
        return DIFFATTN_ERR_NULL;
    const void* ptr[diffattn::BWD_TENSORS] = {q1, k1, q2, k2, v, dy, dq1, dk1, dq2, dk2, dv};
    for (const void* p : ptr)
        if (!aligned16(p)) return DIFFATTN_ERR_ALIGN;
    if (!aligned16(saved)) return DIFFATTN_ERR_ALIGN;
    const size_t need = diffattn_bwd_workspace_bytes(B, H, N, d);
    if (!workspace || workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return DIFFATTN_ERR_ALIGN;
    Footprint f[diffattn::BWD_TENSORS];
    diffattn::BwdStrides G;
    for (int k = 0; k < diffattn::BWD_TENSORS; ++k) {
        const bool wide = k == diffattn::G_V || k == diffattn::G_DY || k == diffattn::G_DV;
        const bool buffered = k <= diffattn::G_V;   // q1, k1, q2, k2, v are read through buffer offsets
        st = strided_tensor(ptr[k], B, H, N, wide ? 128 : 64, strides + 3 * k, buffered, &f[k]);
        if (st) return st;
        G.b[k] = strides[3 * k];
        G.h[k] = strides[3 * k + 1];
        G.n[k] = strides[3 * k + 2];
    }
    for (int k = diffattn::G_DQ1; k <= diffattn::G_DV; ++k)
        if (!one_to_one(B, H, N, k == diffattn::G_DV ? 128 : 64, G.b[k], G.h[k], G.n[k])) return DIFFATTN_ERR_ALIAS;
    // Inputs: q1, k1, q2, k2, v, dy and saved (may overlap one another).  Outputs: the five gradients, dlambda and
    // the workspace (must not overlap one another or any input).
    const Footprint ins[7] = {f[0], f[1], f[2], f[3], f[4], f[5],
                              dense_footprint(saved, diffattn_train_saved_bytes(B, H, N, d))};
    const Footprint outs[7] = {f[6], f[7], f[8], f[9], f[10], dense_footprint(dlambda, (size_t)H * sizeof(float)),
                               dense_footprint(workspace, need)};
    for (int i = 0; i < 7; ++i) {
        for (const Footprint& in : ins)
            if (!disjoint(outs[i], in)) return DIFFATTN_ERR_ALIAS;
        for (int j = i + 1; j < 7; ++j)
            if (!disjoint(outs[i], outs[j])) return DIFFATTN_ERR_ALIAS;
    }
    if (lambda_heads) {
        if (((uintptr_t)lambda_heads & 3u) != 0) return DIFFATTN_ERR_ALIGN;
        const Footprint l = dense_footprint(lambda_heads, (size_t)H * sizeof(float));
        for (const Footprint& o : outs)
            if (!disjoint(l, o)) return DIFFATTN_ERR_ALIAS;
        ep.lambda_heads = lambda_heads;
        ep.heads = (int)H;
    }
    return hip_status(diffattn::launch_bwd_bf16_d64(
        (const uint16_t*)q1, (const uint16_t*)k1, (const uint16_t*)q2, (const uint16_t*)k2, (const uint16_t*)v,
        (const uint16_t*)dy, (const float*)saved, (uint16_t*)dq1, (uint16_t*)dk1, (uint16_t*)dq2, (uint16_t*)dk2,
        (uint16_t*)dv, dlambda, B, H, N, causal, ep, G, workspace, (hipStream_t)stream));
}

}  // extern "C"
