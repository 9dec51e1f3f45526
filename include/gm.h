/*
 * gm.h -- C ABI of the Graph Machine sparse-layer path for AMD MI355X (gfx950).
 *
 * Two stages of a Graph Machine sparse layer, forward and backward, as
 * described on the pages about the Graph Machine (arXiv 2609.02881):
 *   SER  sparse edge referral: A' = Sparsify_s1(A1 A2) over two-hop paths
 *        ("Graph Machine: Towards Better Pretraining via Edges", ai.info,
 *        Key Contributions 3 and Methodology in Plain English);
 *   SEA  sparse edge attention: softmax over the edge slots of
 *        scale * q.k + ln w (product of experts), weighted sum of values
 *        (same page, Key Contributions 3 and Methodology);
 *   backward passes through the soft edge weights only; indices get no
 *   gradient ("Graph Machine" news article on rit.work, section on what was
 *   done; ai.info Methodology).
 *
 * Conventions shared by every call
 *   - Tensors are dense, row-major, contiguous, and live in device memory
 *     owned by the caller.  The library never allocates or frees memory;
 *     scratch space is passed in as a workspace where a call needs one.
 *   - A "unit" is one (batch b, token i, KV head h).  Edge tensors hold one
 *     row of s slots per unit: idx[B][n][hkv][s] int32, w[B][n][hkv][s] fp32.
 *     Indices are local to the sequence and causal: 0 <= idx <= i.  A slot
 *     with w == 0 is padding (index 0 is the padding token that absorbs
 *     missing edges); w must be >= 0 and finite.  Indices are NOT range
 *     checked on the device: an index outside [0, i] reads or writes outside
 *     the row and is undefined behaviour; gm_check_edges is the validator.
 *   - q, o, dout, dq are [B][n][hq][d]; k, v, dk, dv are [B][n][hkv][d].
 *     Query head hq uses KV head hq / (hq_count / hkv) (grouped heads).
 *   - Every call is asynchronous on `stream` (NULL = the null stream), and
 *     every output is fully overwritten.  Shapes, pointers and alignment are
 *     checked on the host first; on any error the call returns a non-zero
 *     status and launches nothing.  Kernel launch failures return
 *     GM_ERR_HIP.
 *   - Limits: B, n, hkv >= 0 (zero sizes are a no-op), B*n*hkv < 2^31,
 *     1 <= s <= 64, s2*s3 <= 64, d in {16, 32, 64, 128, 256}, hq % hkv == 0
 *     (any group size G = hq / hkv; G in {1, 2, 4, 8, 16} takes the row
 *     kernels, other sizes general kernels; gm_decode_step takes
 *     G in {1, 2, 4, 8, 16} only); activation pointers 16-byte aligned,
 *     edge pointers 4-byte aligned.
 *   - Determinism: gm_ser_forward, gm_sea_forward and gm_sea_backward are
 *     bitwise deterministic (the backward sums every dk/dv row over its
 *     incoming edges in ascending edge-id order).  gm_ser_backward
 *     accumulates in fp64, in an order that may vary, and rounds once, so a
 *     result differs between runs only when the fp64 sums straddle an fp32
 *     rounding boundary.
 */
#ifndef GM_H
#define GM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GM_OK = 0,
    GM_ERR_NULL = 1,         /* a required pointer is NULL                  */
    GM_ERR_SHAPE = 2,        /* a size is negative, zero where not allowed,
                                or the product overflows                     */
    GM_ERR_UNSUPPORTED = 3,  /* s, d, dtype or head ratio outside the limits */
    GM_ERR_WORKSPACE = 4,    /* workspace missing or too small               */
    GM_ERR_HIP = 5,          /* a HIP launch or runtime call failed          */
    GM_ERR_ALIGN = 6,        /* a pointer is not aligned as required         */
    GM_ERR_ALIAS = 7,        /* an output overlaps an input it must not      */
    GM_ERR_TOO_LARGE = 8,    /* the sizes need more than the fixed scratch of
                                gm_sea_backward_noalloc                       */
    GM_STATUS_RANGE = 0x7fffffff   /* not a status: gives the type the range of
                                      int, so that any value a caller passes
                                      (e.g. to gm_status_string) is valid */
} gm_status;

/* GM_DTYPE_RANGE is not a dtype: it gives the type the range of int, so that
   the library can reject any value a caller passes (GM_ERR_UNSUPPORTED). */
typedef enum { GM_F32 = 0, GM_BF16 = 1, GM_DTYPE_RANGE = 0x7fffffff } gm_dtype;

/*
 * Sparse edge referral, forward: A' = Sparsify_s1(A1 A2)
 * (ai.info Key Contributions 3; Methodology: the first leg's indices fetch
 * the second leg's indices and weights, then a hard cut to the s1 largest).
 *   in   idx1, w1  [B][n][hkv][s2]  leg 1 (row i of A1)
 *        idx2, w2  [B][n][hkv][s3]  leg 2 (row j of A2); may equal leg 1
 *   out  idx_out, w_out [B][n][hkv][s1]  must not overlap the legs
 * For unit (b,i,h): every path i -> j = idx1[i,a] -> m = idx2[j,c] has weight
 * w1[i,a] * w2[j,c]; paths to the same m are merged by summing (in double,
 * in (a, c) order), the sum is rounded to fp32, and the s1 targets of largest
 * positive weight are kept, equal weights ordered by lower index.  Slots are
 * written in that order; unused slots get (0, 0.0f).  Requires s2*s3 <= 64.
 *   out  paths [B][n][hkv] uint64, optional (NULL: not written; only for
 *        s1, s2, s3 <= 4, else GM_ERR_UNSUPPORTED; 8-byte aligned,
 *        overlapping nothing): the path map of each unit, 4 bits per path
 *        k = 4a + c at bits [4k, 4k + 4): the slot of A' that path's target
 *        went to, or 15 when the path has a zero leg weight or its target
 *        was not kept (and for k beyond the s2 x s3 paths, a >= s2 or
 *        c >= s3).  gm_ser_backward takes it to skip regathering the
 *        leg-2 indices and re-reading A'.
 */
gm_status gm_ser_forward(int B, int n, int hkv,
                         const int32_t* idx1, const float* w1, int s2,
                         const int32_t* idx2, const float* w2, int s3,
                         int32_t* idx_out, float* w_out, int s1, uint64_t* paths,
                         hipStream_t stream);

/*
 * Two chained referral steps in one call (ai.info Key Contributions 2: the
 * edge matrix raised to a power, one referral step per factor; Methodology:
 * each step mixes the edges the previous step left):
 *   A1 = Sparsify_s(A0 A0), A2 = Sparsify_s(A1 A1)
 *   in   idx, w            [B][n][hkv][s]  A0, s = 2 or 4 (else
 *                          GM_ERR_UNSUPPORTED)
 *   out  idx_mid, w_mid    [B][n][hkv][s]  A1, optional (both NULL: not
 *                          written; one NULL: GM_ERR_NULL)
 *        idx_out, w_out    [B][n][hkv][s]  A2
 * Every pointer must be aligned to s*4 bytes (GM_ERR_ALIGN) and no output
 * may overlap another array (GM_ERR_ALIAS).  A1 and A2 are bitwise what two
 * gm_ser_forward calls with s1 = s2 = s3 = s and both legs equal give.
 * One launch: each unit recomputes the rows of A1 it needs (its own and
 * those at its s targets) instead of waiting for other workgroups to write
 * them, so no A1 round trip through memory is needed.  That is s + 2
 * merges per unit instead of 2: on MI355X it takes about twice as long as
 * the two gm_ser_forward calls (the merges, not memory, bound it), so it is
 * for callers that want A2 without holding A1.
 */
gm_status gm_ser_forward_chain2(int B, int n, int hkv, const int32_t* idx, const float* w,
                                int s, int32_t* idx_mid, float* w_mid,
                                int32_t* idx_out, float* w_out, hipStream_t stream);

/*
 * Sparse edge attention, forward (ai.info Key Contributions 3: edge indices
 * pick the positions that supply keys and values, node factor = scaled
 * query-key score, edge factor = log edge weight, product of experts;
 * Methodology: RoPE omitted).
 *   in   q [B][n][hq][d], k, v [B][n][hkv][d]  dtype dt (fp32 or bf16)
 *        idx, w [B][n][hkv][s1]
 *        scale: multiplies q.k (normally 1/sqrt(d))
 *   out  o [B][n][hq][d] dtype dt
 *        stats [B][hkv][n][E*G + 2][s1] 4-byte words, G = hq/hkv, E = 1 for
 *        bf16 inputs and 2 for fp32 inputs (KV-head-major, so that each
 *        pass writes and reads it in contiguous rows), optional (NULL: not
 *        written; else 16-byte aligned, overlapping nothing): the first
 *        E*G rows of a unit hold, for query head hkv_index*G + g and slot
 *        t (in (g, t) order), p_t / w_t of every live slot, i.e.
 *        exp(scale*q.k[idx_t]) / sum_u w_u exp(scale*q.k[idx_u]), and 0 for
 *        a dead slot, as fp32 (E = 1) or fp64 (E = 2: G*s1 doubles, the
 *        precision the fp32-input backward computes in); row E*G holds idx
 *        (the int32 bits) and row E*G + 1 w, a copy of the unit's edge row.
 *        gm_sea_backward takes it to skip the softmax recomputation (and
 *        the q reads it needs) and reads its edges from the copy.
 * o[hq] = sum_t p_t v[idx_t], p = softmax over live slots (w_t > 0) of
 * scale*q.k[idx_t] + ln w_t; a unit with no live slot gets o = 0.
 * Arithmetic is fp32 for bf16 inputs and fp64 for fp32 inputs.
 */
gm_status gm_sea_forward(int B, int n, int hq, int hkv, int d, gm_dtype dt,
                         float scale, const void* q, const void* k, const void* v,
                         const int32_t* idx, const float* w, int s1, void* o,
                         float* stats, hipStream_t stream);

/*
 * gm_ser_forward then gm_sea_forward on its output, in one call: A' =
 * Sparsify_s1(A1 A2) is written to idx_out / w_out as gm_ser_forward writes
 * it (bitwise), and o (and, when given, stats) as gm_sea_forward writes them
 * for that A' (ai.info Key Contributions 3: referral then attention in a
 * sparse layer).  For bf16, d = 128, s1 = s2 = s3 = 4, 16-byte aligned edge
 * rows and hq / hkv in {1, 2, 4, 8, 16} the two stages run as one kernel
 * (A' stays in registers between them); other shapes run the two stages one
 * after the other.  Arguments (paths as gm_ser_forward's), limits and errors
 * as the two calls; no output may overlap an input or another output.
 */
gm_status gm_ser_sea_forward(int B, int n, int hq, int hkv, int d, gm_dtype dt, float scale,
                             const int32_t* idx1, const float* w1, int s2,
                             const int32_t* idx2, const float* w2, int s3, int s1,
                             const void* q, const void* k, const void* v,
                             int32_t* idx_out, float* w_out, void* o, float* stats,
                             uint64_t* paths, hipStream_t stream);

/*
 * Bytes of device workspace gm_sea_backward needs for these sizes: per-edge
 * softmax coefficients, the in-degree of every K/V row, row offsets and the
 * reverse (target-sorted) edge list.
 */
size_t gm_sea_backward_workspace_bytes(int B, int n, int hq, int hkv, int s1);

/*
 * Sparse edge attention, backward: chain rule of gm_sea_forward with the
 * indices held fixed (rit.work: indices get no gradient, learning goes
 * through the soft edge weights).
 *   in   q, k, v, idx, w, s1, scale as for the forward; dout [B][n][hq][d] dt;
 *        stats: NULL, or what gm_sea_forward wrote for these q, k, idx, w
 *        and scale (16-byte aligned).  The backward then takes
 *        p_t = stats_t * w_t and dl_t / w_t from it instead of recomputing
 *        the scores (in fp64 for fp32 inputs, whose statistics are fp64).
 *        Precision: bf16 inputs are computed in fp32.  For fp32 inputs the
 *        scores, softmax, g - gbar, dq, dw and the dk/dv row sums are fp64;
 *        the per-edge coefficients (scale * dl, p) that the source-token
 *        pass hands to the K/V-row pass are rounded to fp32 in between.
 *   out  dq [B][n][hq][d] fp32, dk, dv [B][n][hkv][d] fp32,
 *        dw [B][n][hkv][s1] fp32; no output may overlap an input.
 *   ws   device workspace of gm_sea_backward_workspace_bytes(...) bytes,
 *        256-byte aligned; its contents on entry do not matter.
 * With g_t = dout.v[idx_t], gbar = sum p_t g_t, dl_t = p_t (g_t - gbar):
 * dq = scale sum_t dl_t k[idx_t]; dk[idx_t] += scale dl_t q;
 * dv[idx_t] += p_t dout; dw_t = sum over the group's query heads of
 * dl_t / w_t.  g_t - gbar is formed as sum over u != t of p_u (g_t - g_u)
 * (rows of more slots than one lane team holds: from the unnormalised sums,
 * (g_t Z - sum_u e_u g_u) / Z), so a single live slot gets exactly 0 and a
 * slot holding nearly all the mass loses little of dw to cancellation, however
 * small its weight.  Padding slots (w = 0) get and pass
 * no gradient.  dk and dv are reduced per K/V row over its incoming edges
 * in ascending edge-id order (a target-sorted pass, no float atomics), so
 * the call is bitwise deterministic.  Also requires B*n*hkv*s1 < 2^31.
 */
gm_status gm_sea_backward(int B, int n, int hq, int hkv, int d, gm_dtype dt,
                          float scale, const void* q, const void* k, const void* v,
                          const int32_t* idx, const float* w, int s1,
                          const void* dout, const float* stats, float* dq, float* dk,
                          float* dv, float* dw, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * gm_sea_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results as
 * gm_sea_backward (bitwise), with the workspace in a fixed array of
 * GM_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The call itself allocates and frees nothing.
 *   - Sizes whose gm_sea_backward_workspace_bytes(...) exceeds
 *     GM_NOALLOC_SCRATCH_BYTES return GM_ERR_TOO_LARGE and launch nothing
 *     (the measured layer, B = 8, n = 4096, 8 KV heads, G = 2, s1 = 4,
 *     needs 32 MiB).
 *   - Every call on one GPU shares that GPU's array: calls that may run at
 *     the same time on one GPU (different streams, or threads) race and
 *     must be ordered by the caller.
 *   - The first call on a GPU looks up the array's device address
 *     (hipGetSymbolAddress, with that GPU current); failure returns
 *     GM_ERR_HIP.  The GPU is the one `stream` belongs to (the current one
 *     for the null stream).
 * Other arguments, checks and errors as gm_sea_backward.
 */
#define GM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gm_status gm_sea_backward_noalloc(int B, int n, int hq, int hkv, int d, gm_dtype dt,
                                  float scale, const void* q, const void* k, const void* v,
                                  const int32_t* idx, const float* w, int s1,
                                  const void* dout, const float* stats, float* dq, float* dk,
                                  float* dv, float* dw, hipStream_t stream);

/*
 * Bytes of device workspace gm_ser_backward needs for these sizes: fp64
 * accumulators for dw1 and dw2 (`aliased` is accepted for symmetry with the
 * call; both layouts need the two arrays).
 */
size_t gm_ser_backward_workspace_bytes(int B, int n, int hkv, int s2, int s3,
                                       int aliased);

/*
 * Sparse edge referral, backward: chain rule of gm_ser_forward with the
 * selection held fixed (ai.info Methodology: gradients reach the kept
 * weights alone).
 *   in   legs as for the forward; idx_out, w_out [B][n][hkv][s1] the A' the
 *        forward produced; dw_out [B][n][hkv][s1] the gradient of w_out;
 *        paths: NULL, or the path map gm_ser_forward wrote for these legs
 *        (s1, s2, s3 <= 4; 8-byte aligned).  With it the source-chunk path
 *        (s2 = s3 = 4) reads each path's slot instead of gathering the
 *        leg-2 indices and comparing them with A' (same results, bitwise).
 *   out  dw1 [B][n][hkv][s2], dw2 [B][n][hkv][s3] fp32.  dw1 == dw2 is
 *        allowed (A' = Sparsify(A A), s2 == s3): the sum of both is written.
 *   ws   device workspace of gm_ser_backward_workspace_bytes(...) bytes,
 *        8-byte aligned (16-byte alignment enables the partial-sum path of
 *        s2 = s3 = 4, s1 = 4 or 2, n <= 4096).
 * For each path (a, c) with w1 > 0 and w2 > 0 whose target equals a
 * retained slot t (w_out_t > 0): dw1[i,a] += dw_out_t w2[j,c] and
 * dw2[j,c] += dw_out_t w1[i,a].  Slots with zero weight get 0.
 */
gm_status gm_ser_backward(int B, int n, int hkv,
                          const int32_t* idx1, const float* w1, int s2,
                          const int32_t* idx2, const float* w2, int s3,
                          const int32_t* idx_out, const float* w_out, int s1,
                          const float* dw_out, const uint64_t* paths, float* dw1, float* dw2,
                          void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * Leg construction (ai.info Methodology, referral paragraph: referral mixes
 * the stored edges into pairs and sparsifies each leg before composing
 * them).  The pages give no mixing formula; reading: a leg is a
 * non-negative mixture of a token's K stored edges with one weight per
 * (KV head, stored slot):
 *   leg[i] = Sparsify_s( sum_k alpha[h][k] * w[i][k] e_{idx[i][k]} )
 * merged in slot order in fp64, then SER's selection rules (top s by fp32
 * weight, ties to the lower index, padding (0, 0)).  Call it once per leg.
 *   in   idx, w [B][n][hkv][K] the stored edges (1 <= K <= 64, causal);
 *        alpha [hkv][K] fp32 >= 0 (a learned parametrization that keeps
 *        it non-negative is the caller's)
 *   out  idx_out, w_out [B][n][hkv][s] (1 <= s <= 64)
 * Bitwise deterministic.  Edge pointers 4-byte aligned; outputs must not
 * overlap inputs.
 */
gm_status gm_leg_mix_forward(int B, int n, int hkv, const int32_t* idx, const float* w, int K,
                             const float* alpha, int s, int32_t* idx_out, float* w_out,
                             hipStream_t stream);

/* Bytes of device workspace gm_leg_mix_backward needs (fp64 partial sums). */
size_t gm_leg_mix_backward_workspace_bytes(int B, int n, int hkv, int K);

/*
 * Leg construction backward, the selection held fixed (only retained leg
 * slots pass gradient, as for SER): for each stored slot k with
 * alpha[h][k] > 0 and w[i][k] > 0 and each retained leg slot t (w_out > 0)
 * with the same index:
 *   dw[i][k] += dleg[i][t] * alpha[h][k]     dalpha[h][k] += dleg[i][t] * w[i][k]
 *   in   idx, w, K, alpha as for the forward; idx_out, w_out, s: its output;
 *        dleg [B][n][hkv][s] fp32
 *   out  dw [B][n][hkv][K], dalpha [hkv][K] fp32, both overwritten
 *   ws   device workspace of gm_leg_mix_backward_workspace_bytes(...)
 *        bytes, 8-byte aligned
 * dalpha is summed in fp64 in a fixed order and rounded once: bitwise
 * deterministic.
 */
gm_status gm_leg_mix_backward(int B, int n, int hkv, const int32_t* idx, const float* w, int K,
                              const float* alpha, const int32_t* idx_out, const float* w_out,
                              int s, const float* dleg, float* dw, float* dalpha, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step of the sparse layer (inference; ai.info "Why This Matters":
 * long-context inference): SER then SEA for the newest token of each of B
 * sequences, against caches of the earlier tokens' edge rows and K/V rows.
 * Per (b, KV head h):
 *   A'_b = Sparsify_s1(A1_b . A2_cache)   as gm_ser_forward for one row: the
 *          token's leg-1 slots a point at cache rows j_a, whose s3 slots give
 *          the two-hop targets; same merge, ranking and padding rules, and
 *          bitwise the weights gm_ser_forward produces for that row
 *   o_b  = SEA(q_b, k_cache, v_cache, A'_b)  as gm_sea_forward for one row
 *   in   idx1, w1 [B][hkv][s2] the token's leg-1 row (indices into the cache);
 *        idx2, w2 [B][T][hkv][s3] the edge cache (leg 2);
 *        q [B][hq][d]; k, v [B][T][hkv][d] the K/V cache, dtype dt (the
 *        token's own row written at its position before the call)
 *   out  idx_out, w_out [B][hkv][s1]; o [B][hq][d] dtype dt
 * Indices must address filled cache rows (not checked on the device; out of
 * range is undefined behaviour).  Limits as gm_ser_forward and
 * gm_sea_forward (T plays n); activation pointers 16-byte aligned, edge
 * pointers 4-byte aligned; no output may overlap an input or another output.
 * One launch; no workspace.
 */
gm_status gm_decode_step(int B, int T, int hq, int hkv, int d, gm_dtype dt, float scale,
                         const int32_t* idx1, const float* w1, int s2,
                         const int32_t* idx2, const float* w2, int s3, int s1,
                         const void* q, const void* k, const void* v,
                         int32_t* idx_out, float* w_out, void* o, hipStream_t stream);

/*
 * Refresh edges from a dense causal attention layer (ai.info Methodology,
 * referral paragraph: optional refresh edges bring in the positions the most
 * recent dense attention layer attends to most).  Per (b, token i, KV head h)
 * with G = hq / hkv query heads q_g in the group:
 *   lse_g = log sum_{j<=i} exp(scale q_g . k_j)
 *   pbar_j = (1/G) sum_g exp(scale q_g . k_j - lse_g),   j <= i
 * The s positions of largest pbar_j (equal values: the lower j first) with
 * weight pbar_j, sorted by weight; slots past the i+1 positions hold (0, 0).
 *   in   q [B][n][hq][d], k [B][n][hkv][d] bf16 (the dense layer's queries
 *        and keys after any position encoding); lse_given != 0: lse holds
 *        the layer's own per-head log-sum-exp (natural log) and only the
 *        selection runs
 *   out  idx_out [B][n][hkv][s] int32, w_out [B][n][hkv][s] fp32 (an edge
 *        tensor as SER and SEA take it); lse [B][n][hq] fp32, written when
 *        lse_given == 0
 * Limits: dt GM_BF16 only; (d, G) in {64: 1,2,4,8; 128: 1,2,4; 256: 1,2};
 * 1 <= s <= 8; scale positive and finite.  q, k 16-byte aligned; lse, idx_out, w_out 4-byte aligned;
 * no output may overlap an input or another output.  Two launches (one with
 * lse_given), except for G = 1 without lse_given: one launch forms lse and
 * keeps the positions of largest score (the same order as pbar when G = 1),
 * and weighs them with the final lse.  No workspace.  Scores are fp32 sums
 * of bf16 products on the matrix cores, so positions whose pbar differ by
 * less than that rounding may come out in either order.
 */
gm_status gm_dense_refresh(int B, int n, int hq, int hkv, int d, gm_dtype dt, float scale,
                           const void* q, const void* k, int s, int lse_given, float* lse,
                           int32_t* idx_out, float* w_out, hipStream_t stream);

/*
 * Debug validator of an edge tensor.  Adds to counts[0] the number of slots
 * whose index lies outside [0, i] or whose weight is negative or not finite,
 * and to counts[1] the number of live slots (w > 0), i.e. the key/value rows
 * SEA reads (ai.info Main Findings, KV access).  counts is device memory of
 * two uint64 the caller zeroes; the call is asynchronous on `stream`.
 */
gm_status gm_check_edges(int B, int n, int hkv, const int32_t* idx,
                         const float* w, int s, unsigned long long* counts,
                         hipStream_t stream);

/* Static text for a status code. */
const char* gm_status_string(gm_status status);

/* ABI version: bumped on any change of the calls above. */
int gm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GM_H */
