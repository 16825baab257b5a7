/*
 * diffattn.h -- C ABI of the MI355X (gfx950) differential attention forward library, libdiffattn.so.
 *
 * Pages this API implements (the operation is restated here, not quoted):
 *   [U] Ultralytics glossary entry "Differential Transformer", section on how differential attention works:
 *       the worked PyTorch example (two query/key halves of width d per head, values of width 2d, two softmax
 *       maps with scores divided by sqrt(d), their difference with weight lambda, times V) and the paragraph
 *       after it (per-head normalisation of the output, then the (1 - lambda_init) scale with
 *       lambda_init(l) = 0.8 - 0.6 exp(-0.3 (l - 1))).
 *   [J] jisaku.com glossary entry "Differential Transformer (Diff Attention)", section "main features /
 *       mechanism" (two query/key pairs, difference of the two softmax maps, learnable lambda).
 *
 * For each batch b, head h and query row i the library computes
 *     a = softmax_j(q1_i . k1_j / sqrt(d)),  b = softmax_j(q2_i . k2_j / sqrt(d))     over the visible keys j
 *     o = sum_j (a_j - lambda * b_j) v_j                                                (2d channels)
 *     layer == 0: out_i = o
 *     layer >= 1: out_i = o / sqrt(mean_c(o_c^2) + 1e-5) * (1 - lambda_init(layer))   (RMS norm, no affine)
 * With `causal` set, key j is visible to query row i when j <= i + (Nk - Nq) (the lower triangle for a square
 * prefill; a single decode query sees the whole cache).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library never allocates, frees or
 *     synchronises.  Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream).  Outputs
 *     are valid once the stream reaches the call; inputs must stay alive until then.
 *   - Layouts are dense row-major ("contiguous"):
 *         prefill: q1, k1, q2, k2 [B][H][N][d];  v, out [B][H][N][2d]
 *         decode:  q1, q2 [B][H][d];  k1, k2 [B][H][L][d];  v [B][H][L][2d];  out [B][H][2d]
 *   - Element type `dtype`: DIFFATTN_BF16 (inputs and output bf16, fp32 accumulation) or DIFFATTN_F32 (fp32
 *     throughout).  Supported: bf16 with d = 64; fp32 with d = 8 or 64.  Anything else -> DIFFATTN_ERR_UNSUPPORTED.
 *   - Every tensor pointer must be 16-byte aligned (the per-head lambda array: 4-byte).  `out` (and the decode
 *     workspace) must not overlap any input.
 *   - Arguments are validated before any HIP call; on error nothing is launched and the status says why.
 *     Nothing is printed and nothing is thrown across the ABI.
 *   - Thread safety: no mutable global state; concurrent calls on different streams are independent.
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum diffattn_dtype { DIFFATTN_BF16 = 0, DIFFATTN_F32 = 1 };

enum diffattn_status {
    DIFFATTN_OK = 0,
    DIFFATTN_ERR_NULL = -1,        /* a required pointer is NULL while there is work to do */
    DIFFATTN_ERR_SHAPE = -2,       /* negative size, decode L == 0, or a size beyond the documented limits */
    DIFFATTN_ERR_UNSUPPORTED = -3, /* (dtype, d) combination not implemented */
    DIFFATTN_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    DIFFATTN_ERR_LAYER = -5,       /* layer < 0 */
    DIFFATTN_ERR_LAMBDA = -6,      /* lambda is NaN or infinite */
    DIFFATTN_ERR_WORKSPACE = -7,   /* workspace NULL or smaller than the entry point's *_workspace_bytes() */
    DIFFATTN_ERR_ALIAS = -8,       /* out or workspace overlaps an input (or each other) */
    DIFFATTN_ERR_HIP = -9          /* the HIP runtime reported an error at launch */
};

/* Largest sequence / cache length accepted: one head's V (L x 2d bf16) must stay below 4 GiB because the kernels
 * address a head through a 32-bit buffer offset. */
#define DIFFATTN_MAX_LEN (1 << 23)

/* Most new tokens per sequence in one diffattn_decode_varlen or diffattn_decode_paged call. */
#define DIFFATTN_MAX_NEW_TOKENS 16

/* Largest page of a paged decode cache (rows). */
#define DIFFATTN_MAX_PAGE_SIZE 65536

/*
 * Prefill (square, Nq = Nk = N): the whole forward pass for B x H heads of N tokens.
 *   q1,k1,q2,k2: [B][H][N][d]; v, out: [B][H][N][2d]; element type `dtype`.
 *   lambda: weight of the second map (finite).  layer: 0 = raw output, >= 1 = normalised and scaled by
 *   1 - lambda_init(layer).  causal: 0 or non-zero.
 * N == 0 or B*H == 0 is a successful no-op.  Returns a diffattn_status.
 */
int diffattn_fwd(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, void *out,
                 int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda, int layer, int causal,
                 void *stream);

/*
 * Decode: one new query token per (b, h) against a cache of L keys (the query is position L - 1, so every key
 * is visible and `causal` has no effect).  Split over the cache, then merged; the split partials live in a
 * caller-provided device workspace of at least diffattn_decode_workspace_bytes(B, H, L, d) bytes (16-byte
 * aligned, not overlapping anything else; its contents on entry are ignored and on exit are unspecified).
 *   q1,q2: [B][H][d]; k1,k2: [B][H][L][d]; v: [B][H][L][2d]; out: [B][H][2d].
 * L == 0 is DIFFATTN_ERR_SHAPE (a softmax over no keys is undefined); B*H == 0 is a no-op.
 * The fp32 path evaluates the single row exactly and uses no workspace (it may be NULL); the workspace size
 * function returns the bf16 requirement for d = 64 and 0 for any other d or for an empty problem.
 */
size_t diffattn_decode_workspace_bytes(int64_t B, int64_t H, int64_t L, int d);
int diffattn_decode(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, void *out,
                    int64_t B, int64_t H, int64_t L, int d, int dtype, float lambda, int layer, int causal,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Per-head lambda variants.  The weight lambda of the second softmax map is learned per layer and may differ per
 * head ([U], the paragraph after the worked example: lambda is a learnable scalar; [J] main features): these two
 * entry points take it as an array instead of one float.  Every other argument, the layouts, the statuses and the
 * stream semantics are those of diffattn_fwd and diffattn_decode.
 *
 *   lambda_heads  DEVICE pointer to H fp32 values, 4-byte aligned; head h of every batch entry uses lambda_heads[h].
 *                 Read by the kernels on `stream`; the caller keeps it alive and unchanged until the call's work
 *                 has finished, and it must not overlap `out` (or the decode workspace).  Its values are not
 *                 inspected on the host: a non-finite entry yields non-finite outputs for that head.
 *   Errors:       DIFFATTN_ERR_NULL if lambda_heads is NULL (and the call has work), DIFFATTN_ERR_ALIGN if it is
 *                 not 4-byte aligned, DIFFATTN_ERR_ALIAS if it overlaps out or the workspace.
 */
int diffattn_fwd_heads(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, void *out,
                       int64_t B, int64_t H, int64_t N, int d, int dtype, const float *lambda_heads, int layer,
                       int causal, void *stream);
int diffattn_decode_heads(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, void *out,
                          int64_t B, int64_t H, int64_t L, int d, int dtype, const float *lambda_heads, int layer,
                          int causal, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Strided prefill (bf16, d = 64): diffattn_fwd with every tensor addressed through element strides, so that
 * q1, k1, q2, k2 and v can be read straight out of packed projection outputs (the pages split one projection into
 * the two query/key halves: [U] worked example) and out written into any row layout.
 *   strides: HOST array of 18 int64 values, for q1, k1, q2, k2, v, out in that order: the batch, head and row
 *            strides in elements.  The feature dimension (d, or 2d for v and out) is contiguous.  Element
 *            (b, h, n, c) of tensor t is at base_t + b*strides[3t] + h*strides[3t+1] + n*strides[3t+2] + c.
 *   Every stride must be >= 0, a multiple of 8 (16-byte rows; else DIFFATTN_ERR_ALIGN), and a row stride at least
 *   the row width.  One head's K1, K2 and V rows, N + 256 of them, must span less than 4 GiB
 *   (else DIFFATTN_ERR_SHAPE).  Outputs must not overlap the inputs' address ranges (bounding boxes), and out's
 *   strides must give every element its own address: ordered by stride, the dimensions of extent > 1 (the row of
 *   2d elements first, stride 1) must each have a stride of at least the previous stride times the previous
 *   extent; otherwise DIFFATTN_ERR_ALIAS (several workgroups would write one element).
 *   lambda / lambda_heads as for diffattn_fwd_train.  Contiguous strides give diffattn_fwd's result bit for bit.
 */
int diffattn_fwd_strided(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, void *out,
                         int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda, const float *lambda_heads,
                         int layer, int causal, const int64_t *strides, void *stream);

/*
 * Split-key prefill (bf16, d = 64, dense tensors as for diffattn_fwd): the same operation ([U] worked example and
 * the paragraph after it) for launches whose B * H * ceil(N / 128) row tiles are too few to fill the GPU (fewer
 * than 512 workgroup slots: few heads, or long rows with one or two heads).  The key range of every row tile is cut
 * into up to 16 ranges handled by separate workgroups (a causal row tile only has the ranges up to its diagonal);
 * each writes its rows' partial softmax states (per map: offset, sum and unnormalised output) to `workspace`, and a
 * second kernel merges each row's states by log-sum-exp and applies the epilogue, as the split decode does.  The
 * split count is the one of least modelled time (the longest range's key loop, memory traffic of the running
 * workgroups and the merge's reads, fitted to measured launches), and may be 1.  The result equals diffattn_fwd's
 * up to rounding (the sums are taken in another order), not bit for bit.
 *   diffattn_fwd_split_workspace_bytes: bytes of workspace the call needs: B*H*N*splits*1040 with the larger
 *     split count of the causal and the non-causal plan, or 0 when neither splits (then the call runs
 *     diffattn_fwd's kernel and reads no workspace) or the shape is unsupported.
 *   lambda / lambda_heads: as for diffattn_fwd_strided (lambda_heads NULL = one lambda for all heads; it must
 *     not overlap out or the workspace).
 *   workspace: device, 16-byte aligned, >= that size, overlapping no input or out (contents on entry ignored; the
 *     call leaves partial states in it).  Calls that overlap in time must use different workspaces.
 *   Errors as for diffattn_fwd; dtype other than bf16 or d != 64 -> DIFFATTN_ERR_UNSUPPORTED; a missing or small
 *   workspace -> DIFFATTN_ERR_WORKSPACE; a workspace overlapping a tensor -> DIFFATTN_ERR_ALIAS.
 */
size_t diffattn_fwd_split_workspace_bytes(int64_t B, int64_t H, int64_t N, int d);
int diffattn_fwd_split(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, void *out,
                       int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda, const float *lambda_heads,
                       int layer, int causal, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Variable-length and multi-token decode (bf16, d = 64).  Each sequence b has a cache of lens[b] valid rows in a
 * cache padded to L rows, and T new tokens (1 <= T <= DIFFATTN_MAX_NEW_TOKENS) that are already the last T of those
 * rows: new token t is position lens[b] - T + t and sees the keys up to and including its own position (the causal
 * reading of the worked example applied to a cache, as for diffattn_decode).
 *   q1, q2: [B][H][T][d];  k1, k2: [B][H][L][d];  v: [B][H][L][2d];  out: [B][H][T][2d].
 *   lens: DEVICE array of B int32 values, 4-byte aligned, or NULL (every sequence uses all L rows).  Each value is
 *         clamped on the device to [T, L]; it is read on `stream` and must not overlap out or the workspace.
 *   lambda / lambda_heads: as for diffattn_fwd_train (lambda_heads NULL = one lambda for all heads).
 *   workspace: >= diffattn_decode_varlen_workspace_bytes(B, H, T, L, d) bytes, 16-byte aligned.
 * Errors as for diffattn_decode; T < 1, T > 16 or L < T is DIFFATTN_ERR_SHAPE; fp32 is DIFFATTN_ERR_UNSUPPORTED.
 * With T = 1 and lens NULL the result equals diffattn_decode (same kernels).
 */
size_t diffattn_decode_varlen_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t L, int d);
int diffattn_decode_varlen(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, void *out,
                           int64_t B, int64_t H, int64_t T, int64_t L, const int32_t *lens, int d, int dtype,
                           float lambda, const float *lambda_heads, int layer, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Strided decode caches (bf16, d = 64): diffattn_decode_varlen with K1, K2 and V read through batch, head and row
 * strides, so a cache kept token-major ([B][L][H][w]) or the key halves and values packed in one buffer (for
 * example [B][L][H][d + d + 2d] straight from a fused projection) is read in place.  The computation is that of
 * diffattn_decode_varlen ([U] worked example: the two query/key halves and the values); only the addressing of
 * cache rows differs.
 *   cache_strides: HOST array of 9 int64 values, for k1, k2, v in that order: the batch, head and row strides in
 *                  elements.  Row r of head h of sequence b of tensor t starts at
 *                  base_t + b*cache_strides[3t] + h*cache_strides[3t+1] + r*cache_strides[3t+2]; its d (or 2d)
 *                  features are contiguous.  Every stride must be >= 0 and a multiple of 8 (16-byte rows; else
 *                  DIFFATTN_ERR_ALIGN), a row stride at least the row width (else DIFFATTN_ERR_SHAPE).
 *   q1, q2, out, T, L, lens, lambda, lambda_heads, layer, workspace: as for diffattn_decode_varlen (q1, q2 and out
 *   contiguous; the workspace size is diffattn_decode_varlen_workspace_bytes(B, H, T, L, d)).
 * Errors as for diffattn_decode_varlen; cache_strides NULL is DIFFATTN_ERR_NULL; out or the workspace overlapping
 * any cache's address range (its bounding box) is DIFFATTN_ERR_ALIAS; the caches may overlap each other.  Dense
 * strides give diffattn_decode_varlen's result bit for bit.
 */
int diffattn_decode_strided(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, void *out,
                            int64_t B, int64_t H, int64_t T, int64_t L, const int32_t *lens,
                            const int64_t *cache_strides, int d, int dtype, float lambda, const float *lambda_heads,
                            int layer, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Paged decode (bf16, d = 64): diffattn_decode_varlen over caches kept in fixed-size pages of a pool shared by all
 * sequences, the layout of a serving cache that grows a page at a time.  The method is the same (the pages fix the
 * computation, not where the cache rows live); only the addressing of cache rows differs.
 *   k1_pages, k2_pages: [num_pages][H][page_size][d];  v_pages: [num_pages][H][page_size][2d].
 *   block_table: DEVICE array [B][max_pages] of int32, 4-byte aligned: logical cache row r of sequence b (every
 *                head) is row r % page_size of page block_table[b * max_pages + r / page_size].  Entries are read
 *                on `stream`, only for rows below the sequence's length, and clamped on the device to
 *                [0, num_pages), so no access leaves the pools; a clamped entry reads that page.
 *   page_size:   a power of two in [16, DIFFATTN_MAX_PAGE_SIZE].  L = max_pages * page_size plays the role of the
 *                padded length of diffattn_decode_varlen (L <= DIFFATTN_MAX_LEN, L >= T).
 *   q1, q2, out, T, lens, lambda, lambda_heads, layer: as for diffattn_decode_varlen (lens NULL = L rows each).
 *   workspace: >= diffattn_decode_paged_workspace_bytes(B, H, T, max_pages, page_size, d) bytes, 16-byte aligned,
 *              overlapping nothing else.
 * Errors as for diffattn_decode_varlen; a page_size that is not a power of two in range, max_pages < 1 or
 * num_pages < 1 is DIFFATTN_ERR_SHAPE; block_table NULL is DIFFATTN_ERR_NULL; a block table or lens not 4-byte
 * aligned is DIFFATTN_ERR_ALIGN; out overlapping any input (pools, table, lens) is DIFFATTN_ERR_ALIAS.  The result
 * equals diffattn_decode_varlen on the cache gathered page by page (same kernels, same split plan for L).
 */
size_t diffattn_decode_paged_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t max_pages, int64_t page_size,
                                             int d);
int diffattn_decode_paged(const void *q1, const void *k1_pages, const void *q2, const void *k2_pages,
                          const void *v_pages, void *out, int64_t B, int64_t H, int64_t T,
                          const int32_t *block_table, int64_t max_pages, int64_t page_size, int64_t num_pages,
                          const int32_t *lens, int d, int dtype, float lambda, const float *lambda_heads, int layer,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Training: a forward that keeps what the backward pass needs, and the backward pass.  The pages describe no
 * backward; it is the chain rule of the forward above (normalisation, the lambda-weighted difference, both
 * softmaxes, the scaled scores), so gradients are those of the exact forward definition.  bf16 with d = 64 only
 * (anything else -> DIFFATTN_ERR_UNSUPPORTED); causal or not; lambda scalar, or per head when lambda_heads is
 * non-NULL (a device array of H floats, as for diffattn_fwd_heads; then `lambda` is ignored).
 *
 * diffattn_train_saved_bytes: size of `saved` for diffattn_fwd_train, B*H*N*1040 bytes (0 if unsupported).
 * diffattn_fwd_train: same output as diffattn_fwd (bit-identical), and writes `saved` (device, 16-byte aligned,
 *   >= diffattn_train_saved_bytes, overlapping nothing else): per query row the two maps' log-sum-exps, the row's
 *   RMS factor and the two maps' outputs before they are combined (fp32; layout private to the library).
 * diffattn_bwd_workspace_bytes: scratch size for diffattn_bwd (0 for an empty problem or unsupported d).
 * diffattn_bwd: given dy = dLoss/dout ([B][H][N][2d] bf16) and the `saved` of the forward call with the same
 *   inputs, lambda, layer and causal flag, writes dq1, dk1, dq2, dk2 ([B][H][N][d] bf16), dv ([B][H][N][2d] bf16)
 *   and dlambda (device, H floats, 4-byte aligned: dLoss/dlambda of each head, summed over the batch; for one
 *   lambda shared by all heads, sum the H values).  All gradients are overwritten, not accumulated.
 *   workspace: device, 256-byte aligned, >= diffattn_bwd_workspace_bytes (contents on entry ignored).
 *   Outputs, dlambda and workspace must not overlap each other or any input.  N == 0 writes zeros to dlambda;
 *   B*H == 0 is a no-op.  Errors as for diffattn_fwd, plus DIFFATTN_ERR_WORKSPACE for a missing or small
 *   workspace / saved buffer.
 */
size_t diffattn_train_saved_bytes(int64_t B, int64_t H, int64_t N, int d);
int diffattn_fwd_train(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, void *out,
                       int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda, const float *lambda_heads,
                       int layer, int causal, void *saved, size_t saved_bytes, void *stream);
size_t diffattn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int d);
int diffattn_bwd(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, const void *dy,
                 const void *saved, void *dq1, void *dk1, void *dq2, void *dk2, void *dv, float *dlambda, int64_t B,
                 int64_t H, int64_t N, int d, int dtype, float lambda, const float *lambda_heads, int layer,
                 int causal, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Strided training (bf16, d = 64): diffattn_fwd_train and diffattn_bwd with every caller tensor addressed through
 * element strides, so that q1, k1, q2, k2 and v are read straight out of packed projection outputs (as for
 * diffattn_fwd_strided) and the five gradients written straight into the matching packed gradient buffer.  `saved`,
 * the workspace and dlambda keep the dense layouts of the unstrided calls.
 *   diffattn_fwd_train_strided: strides is a HOST array of 18 int64 values for q1, k1, q2, k2, v, out, laid out and
 *     checked as for diffattn_fwd_strided; writes the same out and `saved` as diffattn_fwd_train on dense copies.
 *   diffattn_bwd_strided: strides is a HOST array of 33 int64 values for q1, k1, q2, k2, v, dy, dq1, dk1, dq2, dk2,
 *     dv in that order (batch, head and row strides in elements per tensor; rows of d or 2d contiguous elements).
 *     Every stride must be >= 0 and a multiple of 8 (else DIFFATTN_ERR_ALIGN) and each row stride at least the row
 *     width; one head's q1, k1, q2, k2 and v rows, N + 256 of them, must span less than 4 GiB (else
 *     DIFFATTN_ERR_SHAPE).  Gives diffattn_bwd's results on dense copies bit for bit.
 *   Aliasing: outputs (and, for the backward, the gradients, dlambda and the workspace among themselves) must not
 *   share a byte with each other or with any input.  Two strided tensors count as disjoint when their bounding boxes
 *   are, or when their rows fall in different residue classes modulo the gcd of all their byte strides (for example
 *   the column slices of one packed buffer); anything else that overlaps is DIFFATTN_ERR_ALIAS.  Each output (out,
 *   and each gradient) must also give every one of its own elements a distinct address, by the rule stated for
 *   diffattn_fwd_strided's out; otherwise DIFFATTN_ERR_ALIAS.
 */
int diffattn_fwd_train_strided(const void *q1, const void *k1, const void *q2, const void *k2, const void *v,
                               void *out, int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda,
                               const float *lambda_heads, int layer, int causal, const int64_t *strides, void *saved,
                               size_t saved_bytes, void *stream);
int diffattn_bwd_strided(const void *q1, const void *k1, const void *q2, const void *k2, const void *v,
                         const void *dy, const void *saved, void *dq1, void *dk1, void *dq2, void *dk2, void *dv,
                         float *dlambda, int64_t B, int64_t H, int64_t N, int d, int dtype, float lambda,
                         const float *lambda_heads, int layer, int causal, const int64_t *strides, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * Decode without allocation, for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): diffattn_decode with the split partials kept in a scratch array
 * that the library holds in each GPU's memory (DIFFATTN_NOALLOC_SCRATCH_BYTES, from the first call on that GPU
 * until the process ends) instead of a caller workspace.  The call itself allocates nothing.
 *   Arguments, layouts, results and errors as for diffattn_decode; the call must need at most
 *   DIFFATTN_NOALLOC_SCRATCH_BYTES of partials (diffattn_decode_workspace_bytes(B, H, L, d); for example B = 64,
 *   H = 16 up to L = 61440), else DIFFATTN_ERR_WORKSPACE before any HIP call.  The partials are fully rewritten by
 *   every call (no state is carried between calls).  All calls on one GPU share its array: calls that may overlap
 *   in time on one GPU (different streams, or threads) race and must be serialised by the caller.  Results are bit
 *   for bit those of diffattn_decode.  The first call on a GPU, with that GPU current, looks up the array's device
 *   address (DIFFATTN_ERR_HIP if that fails).
 */
#define DIFFATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
int diffattn_decode_noalloc(const void *q1, const void *k1, const void *q2, const void *k2, const void *v, void *out,
                            int64_t B, int64_t H, int64_t L, int d, int dtype, float lambda, int layer, int causal,
                            void *stream);

/* lambda_init(layer) = 0.8 - 0.6 exp(-0.3 (layer - 1)) in double, for layer >= 1 ([U]); NaN for layer < 1. */
double diffattn_lambda_init(int layer);

/* Static description of a status code (never NULL). */
const char *diffattn_status_str(int status);

/* ABI version: bumped on any incompatible change. */
int diffattn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DIFFATTN_H */
