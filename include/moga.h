/*
 * moga.h -- C ABI of the MoGA (Mixture-of-Groups Attention) forward hot path,
 * its spatial-temporal group attention branches and its training backward,
 * for AMD Instinct MI355X (gfx950).
 *
 * Source of the operations: the page "MoGA: Mixture-of-Groups Attention for
 * End-to-End Long Video Generation" (architecture explainer of arXiv
 * 2510.18692).  Section names below refer to that page.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises; every launch goes to `stream`
 *    (a hipStream_t passed as void*; NULL = the null stream) and returns
 *    without waiting.  Scratch memory ("workspace") is caller-allocated, sized
 *    by moga_workspace_bytes().
 *  - bf16 tensors are passed as void* holding IEEE bfloat16 values.  Every
 *    bf16 result is rounded to nearest-even from float32.
 *  - Token tensors Q, K, V, Q_hat, K_hat, V_hat, O_hat and O are contiguous
 *    [N, H, D] (token-major, then head, then channel).  X is [N, d_model];
 *    W_r is [M, d_model] (one prototype per row).
 *  - Group ids are 0-based int32.  cu_seqlens is int32 [M+1] with
 *    cu_seqlens[0] = 0, cu_seqlens[M] = N; an empty group repeats an entry.
 *  - Supported ranges: 1 <= M <= 64; D in {64, 128}; 1 <= H; H*D <= 8192;
 *    1 <= N < 2^31; d_model a positive multiple of 32.
 *  - Return value: MOGA_OK (0) or a negative moga_status.  Argument errors are
 *    found on the host before anything is launched, and then no output buffer
 *    is touched.  Faults inside kernels surface at the caller's next
 *    synchronisation.  Inputs must be finite; group ids outside [0, M) are a
 *    precondition violation and are not checked on the device.
 *  - Calls on different streams may run concurrently; each call only reads
 *    its inputs and writes its outputs and workspace.
 */
#ifndef MOGA_H_
#define MOGA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moga_status {
  MOGA_OK = 0,
  MOGA_ERR_NULL = -1,        /* a required pointer is NULL */
  MOGA_ERR_SHAPE = -2,       /* a size is out of range or sizes disagree */
  MOGA_ERR_UNSUPPORTED = -3, /* a valid but unsupported configuration (e.g. D = 96) */
  MOGA_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than moga_workspace_bytes() */
  MOGA_ERR_HIP = -5          /* the HIP runtime refused a launch */
} moga_status;

typedef enum moga_op {
  MOGA_OP_ROUTE = 0,
  MOGA_OP_PERMUTE = 1,
  MOGA_OP_GROUP_ATTENTION = 2,
  MOGA_OP_UNPERMUTE = 3,
  MOGA_OP_STGA_ATTENTION = 4,
  MOGA_OP_BALANCE_STATS = 5,
  MOGA_OP_ROUTE_BACKWARD = 6,     /* pass d_model as D */
  MOGA_OP_ATTENTION_BACKWARD = 7
} moga_op;

/*
 * moga_route -- router scores, hard assignment and gate for every token.
 *   Section "MoGA Router": r = x W_r (+ optional bias), p(i|x) = softmax(r)_i
 *   (Eq. 3), g(x) = argmax_i p(i|x); Algorithm 1 step 1.  The gate is
 *   p(g(x)|x) = 1 / sum_j exp(r_j - r_g), used by the MoGA output equation
 *   ("Grouped Attention").  Scores are accumulated in float32; the argmax is
 *   taken on the float32 scores, ties going to the lowest group index.
 *   X        bf16 [N, d_model]
 *   Wr       bf16 [M, d_model]
 *   bias     float [M] or NULL (no bias)
 *   group_id int32 [N]  (output)
 *   gate     float [N]  (output)
 *   ws, ws_bytes  workspace of moga_workspace_bytes(MOGA_OP_ROUTE, ...) = 0
 *            bytes: the route needs none, so ws may be NULL; the arguments
 *            keep the signature of the other steps.
 */
int moga_route(const void* X, const void* Wr, const float* bias,
               int64_t N, int32_t d_model, int32_t M,
               int32_t* group_id, float* gate, void* ws, size_t ws_bytes, void* stream);

/*
 * moga_permute -- make every group contiguous (Algorithm 1 step 2).
 *   Groups are laid out in increasing id; inside a group tokens keep their
 *   original order (stable counting sort).
 *   group_id   int32 [N] (input, values in [0, M))
 *   Q, K, V    bf16 [N, H, D] (inputs)
 *   Qp, Kp, Vp bf16 [N, H, D] (outputs): Qp[j] = Q[perm[j]], likewise K, V
 *   perm       int32 [N]   (output): original token of permuted row j
 *   cu_seqlens int32 [M+1] (output): group boundaries in permuted order
 *   max_seqlen int32 [1]   (output, device scalar): largest group size
 *   ws         workspace of at least moga_workspace_bytes(MOGA_OP_PERMUTE, N, M, H, D) bytes
 *   Q, K, V, Qp, Kp, Vp may ALL be NULL: then only perm, cu_seqlens and
 *   max_seqlen are produced (H and D are then ignored).
 */
int moga_permute(const int32_t* group_id, const void* Q, const void* K, const void* V,
                 int64_t N, int32_t H, int32_t D, int32_t M,
                 void* Qp, void* Kp, void* Vp, int32_t* perm, int32_t* cu_seqlens,
                 int32_t* max_seqlen, void* ws, size_t ws_bytes, void* stream);

/*
 * moga_group_attention -- exact softmax attention inside every group
 *   (Eq. 1 restricted to a group; Algorithm 1 step 3), non-causal, each token
 *   attending to itself and every other token of its group, for every head.
 *   Deterministic: the same inputs give the same bits on every call.
 *   Qp, Kp, Vp  bf16 [N, H, D], rows grouped as described by cu_seqlens
 *   cu_seqlens  int32 [M+1] (device)
 *   softmax_scale  > 0, or <= 0 for 1/sqrt(D)
 *   Op          bf16 [N, H, D] (output, permuted order, no gate)
 *   ws          workspace of at least moga_workspace_bytes(MOGA_OP_GROUP_ATTENTION, N, M, H, D)
 *   bf16 MFMA products and float32 accumulation.  The Q operand carries the
 *   softmax scale (in log2 units, rounded to bf16 once per element) and the
 *   float32 softmax runs against a per-row exponent offset fixed before the
 *   key loop: none when the row's first 32 scores are moderate, else their
 *   maximum.  A work item whose denominator leaves [2^-64, 2^64) or whose
 *   float32 accumulator is not finite is recomputed against each row's exact
 *   maximum plus log2 of its exact sum, so every weight is at most 1 and the
 *   accumulator stays within the magnitude of the values: for any finite
 *   input the result is the softmax average of the group's values.
 */
int moga_group_attention(const void* Qp, const void* Kp, const void* Vp,
                         const int32_t* cu_seqlens, int64_t N, int32_t H, int32_t D,
                         int32_t M, float softmax_scale, void* Op,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * moga_group_attention_unpermute -- moga_group_attention and moga_unpermute
 *   in one kernel (MoGA output equation; Algorithm 1 steps 3 and 4): the
 *   attention of permuted row j is written straight to its original token,
 *   O[perm[j]] = beta * O[perm[j]] + gate[perm[j]] * Attn(j), without the
 *   intermediate O_hat.  Arguments as in the two calls it replaces; ws as for
 *   MOGA_OP_GROUP_ATTENTION.  beta = 0 does not read O.
 */
int moga_group_attention_unpermute(const void* Qp, const void* Kp, const void* Vp,
                                   const int32_t* cu_seqlens, const int32_t* perm, const float* gate,
                                   int64_t N, int32_t H, int32_t D, int32_t M, float softmax_scale,
                                   float beta, void* O, void* ws, size_t ws_bytes, void* stream);

/*
 * moga_permute_vt -- moga_permute with V written transposed per head, the
 *   layout moga_group_attention_unpermute_vt reads (Algorithm 1 step 2).
 *   Qp, Kp   bf16 [N, H, D] (outputs) as in moga_permute
 *   Vt       bf16 [H, D, ldv] (output), ldv = N rounded up to a multiple of
 *            64, plus 64: Vt[h][d][j] = V[perm[j]][h][d] for j < N and 0 for
 *            N <= j < ldv; 16-byte aligned.  The padding lets every 64-key
 *            tile of the attention read whole rows.
 *   Other arguments, workspace and errors as in moga_permute.  K, V, Kp and
 *   Vt are required; Q and Qp are either both given (Q is gathered) or both
 *   NULL (only K and V are gathered, for moga_group_attention_unpermute_vtq;
 *   one of the two alone is MOGA_ERR_NULL).  N <= 2^23 - 128
 *   (MOGA_ERR_UNSUPPORTED beyond): the attention kernel addresses one head's
 *   V^T rows with 32-bit offsets.
 */
int moga_permute_vt(const int32_t* group_id, const void* Q, const void* K, const void* V,
                    int64_t N, int32_t H, int32_t D, int32_t M,
                    void* Qp, void* Kp, void* Vt, int32_t* perm, int32_t* cu_seqlens,
                    int32_t* max_seqlen, void* ws, size_t ws_bytes, void* stream);

/*
 * moga_permute_vt_noalloc -- moga_permute_vt for callers that cannot allocate
 *   device memory (code under HIP graph capture, tight serving loops,
 *   harnesses that forbid hipMalloc): the same operation, arguments and
 *   outputs, without the workspace.  The counting sort's scratch (8 * M *
 *   ceil(N / 1024) bytes of block counts and offsets) lives in a fixed 1 MiB
 *   device array inside the library, one copy per GPU, held until the
 *   process ends; sizes that need more return MOGA_ERR_WORKSPACE (M = 64
 *   allows N <= 2^21, M = 16 every N the transposed-V path supports).  The
 *   first call on a device looks that device's copy up, with the device
 *   current (MOGA_ERR_HIP if the lookup fails); no call allocates or frees.
 *   Every entry of the scratch a call reads is written earlier in the same
 *   call, so nothing needs clearing between calls, but all calls on one GPU
 *   share the array: calls that overlap in time on one GPU (several streams
 *   or host threads) race and must be serialised.
 */
int moga_permute_vt_noalloc(const int32_t* group_id, const void* Q, const void* K, const void* V,
                            int64_t N, int32_t H, int32_t D, int32_t M,
                            void* Qp, void* Kp, void* Vt, int32_t* perm, int32_t* cu_seqlens,
                            int32_t* max_seqlen, void* stream);

/*
 * moga_group_attention_unpermute_vt -- moga_group_attention_unpermute with
 *   V given transposed (Vt [H, D, ldv] as written by moga_permute_vt,
 *   padding included; MoGA output equation, Algorithm 1 steps 3 and 4).  Same
 *   result, up to float32 summation order, as the row layout: in LDS a
 *   channel's 8 consecutive keys are one 16-byte read, where rows need two
 *   transposing reads per MFMA operand.  Qp, Kp bf16 [N, H, D]; other
 *   arguments, workspace and errors as in moga_group_attention_unpermute;
 *   N <= 2^23 - 128.
 */
int moga_group_attention_unpermute_vt(const void* Qp, const void* Kp, const void* Vt,
                                      const int32_t* cu_seqlens, const int32_t* perm, const float* gate,
                                      int64_t N, int32_t H, int32_t D, int32_t M, float softmax_scale,
                                      float beta, void* O, void* ws, size_t ws_bytes, void* stream);

/*
 * moga_group_attention_unpermute_vtq -- moga_group_attention_unpermute_vt
 *   with the queries read in original token order (MoGA output equation,
 *   Algorithm 1 steps 3 and 4): Q is the UNPERMUTED bf16 [N, H, D] tensor and
 *   query j of the permuted order is token perm[j], so moga_permute_vt may
 *   skip the Q gather (Q = Qp = NULL there).  Kp bf16 [N, H, D] and
 *   Vt [H, D, ldv] as written by moga_permute_vt.  Each query row is read
 *   once per work item, so reading it through perm costs one index load,
 *   where a gathered copy costs a read and a write of every row.
 *   O[n] = beta * O[n] + gate[n] * Attn(n); same result, bit for bit, as
 *   moga_group_attention_unpermute_vt on the gathered Qp.  Other arguments,
 *   workspace and errors as there; O must not alias Q, Kp or Vt.
 */
int moga_group_attention_unpermute_vtq(const void* Q, const void* Kp, const void* Vt,
                                       const int32_t* cu_seqlens, const int32_t* perm, const float* gate,
                                       int64_t N, int32_t H, int32_t D, int32_t M, float softmax_scale,
                                       float beta, void* O, void* ws, size_t ws_bytes, void* stream);

/*
 * moga_group_attention_fused -- the gated group attention read in place
 *   (gather on load; MoGA output equation, Algorithm 1 steps 2 to 4 after the
 *   sort): Q, K, V are the ORIGINAL-order tensors bf16 [N, H, D], and
 *   permuted row j of a group is read from token perm[j], so no gathered
 *   copies are needed (moga_permute may be called with Q = K = V = NULL).
 *   O[n] = beta * O[n] + gate[n] * Attn(n) for every token n.
 *   cu_seqlens, perm as produced by moga_permute; gate float32 [N]; ws as for
 *   MOGA_OP_GROUP_ATTENTION.  beta = 0 does not read O.  O must not alias
 *   Q, K or V.
 */
int moga_group_attention_fused(const void* Q, const void* K, const void* V,
                               const int32_t* cu_seqlens, const int32_t* perm, const float* gate,
                               int64_t N, int32_t H, int32_t D, int32_t M, float softmax_scale,
                               float beta, void* O, void* ws, size_t ws_bytes, void* stream);

/*
 * moga_unpermute -- gate and return rows to original order
 *   (MoGA output equation in "Grouped Attention"; Algorithm 1 step 4):
 *   O[perm[j]] = beta * O[perm[j]] + gate[perm[j]] * Op[j]  (float32 math).
 *   beta = 0 overwrites O (its old contents are not read); beta != 0
 *   accumulates, e.g. onto an STGA result.
 *   Op bf16 [N, H, D]; perm int32 [N]; gate float [N]; O bf16 [N, H, D] (in/out).
 *   Needs no workspace.
 */
int moga_unpermute(const void* Op, const int32_t* perm, const float* gate,
                   int64_t N, int32_t H, int32_t D, float beta, void* O, void* stream);

/*
 * moga_stga_attention -- static local window attention (section "Spatial-
 *   Temporal Group Attention (STGA)"): tokens are frame-major,
 *   n = (t * Hs + y) * Ws + x with N = T * Hs * Ws, and token n belongs to the
 *   static group (t / win_t, y / tile_h, x / tile_w).  Softmax attention runs
 *   inside each static group, on the original token order, without a gate:
 *   O[n] = beta * O[n] + alpha * STGA(n)   (beta = 0: O is not read).
 *   Q, K, V bf16 [N, H, D]; O bf16 [N, H, D] (in/out).
 *   win_t, tile_h, tile_w must divide T, Hs, Ws; the group size
 *   win_t * tile_h * tile_w must be at most 2^20.
 *   ws, ws_bytes  workspace of moga_workspace_bytes(MOGA_OP_STGA_ATTENTION, ...)
 *   = 0 bytes: the static windows need none, so ws may be NULL.
 */
int moga_stga_attention(const void* Q, const void* K, const void* V,
                        int32_t T, int32_t Hs, int32_t Ws, int32_t win_t, int32_t tile_h,
                        int32_t tile_w, int32_t H, int32_t D, float softmax_scale,
                        float alpha, float beta, void* O, void* ws, size_t ws_bytes, void* stream);

/*
 * moga_stga_shot_attention -- the shot-aware STGA branch (section "Spatial-
 *   Temporal Group Attention (STGA)": frames of different shots never share a
 *   temporal group; keys and values, not queries, are augmented with latent
 *   frames of the adjacent shots).  Frame-major tokens as in
 *   moga_stga_attention.  Every shot [shot_start[s], shot_start[s+1]) is cut
 *   into windows of win_t frames, the last one shorter if the shot length is
 *   not a multiple of win_t.  The queries of a window are its frames' tokens
 *   inside one tile_h x tile_w spatial tile; its keys and values are those
 *   tokens, plus the same tile of the previous shot's last `augment` frames
 *   for the shot's first window and of the next shot's first `augment`
 *   frames for the shot's last window (clipped to those shots; augment = 0
 *   turns augmentation off, 0 <= augment <= 64).
 *   O[n] = beta * O[n] + alpha * STGA(n).
 *   shot_start: DEVICE int32 [n_shots + 1], 0 = shot_start[0] < ... <
 *   shot_start[n_shots] = T (not checked on the host; boundaries outside
 *   that order give unspecified output for the affected frames, never an
 *   out-of-bounds access).  tile_h, tile_w must divide Hs, Ws and
 *   (win_t + 2 * augment) * tile_h * tile_w must be at most 2^20.
 *   ws: device workspace of moga_stga_shot_workspace_bytes(T, n_shots, win_t)
 *   bytes (the window table, rebuilt on every call).
 */
int moga_stga_shot_attention(const void* Q, const void* K, const void* V,
                             int32_t T, int32_t Hs, int32_t Ws, const int32_t* shot_start,
                             int32_t n_shots, int32_t win_t, int32_t tile_h, int32_t tile_w,
                             int32_t augment, int32_t H, int32_t D, float softmax_scale,
                             float alpha, float beta, void* O, void* ws, size_t ws_bytes,
                             void* stream);

/* moga_stga_shot_workspace_bytes -- workspace of moga_stga_shot_attention;
 *   0 for invalid sizes.  Host-only, no device call. */
size_t moga_stga_shot_workspace_bytes(int32_t T, int32_t n_shots, int32_t win_t);

/*
 * moga_balance_stats -- router balance statistics (section "Group Balancing
 *   Loss: Preventing Router Collapse", Eq. 6): F[i] = #{n : group_id[n] = i} / N,
 *   P[i] = (sum of gate[n] over tokens with group_id[n] = i) / N, and
 *   loss[0] = alpha * M * sum_i F[i] * P[i].  F, P float [M]; loss float [1]
 *   (device).  Sums are reduced in a fixed order, so results are
 *   reproducible bit for bit.  ws: moga_workspace_bytes(MOGA_OP_BALANCE_STATS, ...).
 */
int moga_balance_stats(const int32_t* group_id, const float* gate, int64_t N, int32_t M, float alpha,
                       float* F, float* P, float* loss, void* ws, size_t ws_bytes, void* stream);

/*
 * ---- Backward pass ----
 * Gradients of L = sum(O * dO) for the MoGA output O[n] = gate[n] * SA(n)
 * ("Grouped Attention" section: the gate p(g(x)|x) is the router's gradient
 * path, the hard argmax has none).  A training step runs
 *   moga_route -> moga_permute -> moga_group_attention_train (saves Op, lse)
 *   -> moga_unpermute (O) ... and back:
 *   moga_unpermute_backward -> moga_group_attention_backward -> moga_route_backward.
 */

/*
 * moga_group_attention_train -- moga_group_attention that also saves, for the
 *   backward pass, lse[h][j] = log sum_k exp(scale * q_jh . k_kh) over row j's
 *   group (natural log), float [H, N] (head-major, permuted rows).  Other
 *   arguments and ws as moga_group_attention.
 */
int moga_group_attention_train(const void* Qp, const void* Kp, const void* Vp,
                               const int32_t* cu_seqlens, int64_t N, int32_t H, int32_t D,
                               int32_t M, float softmax_scale, void* Op, float* lse,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * moga_unpermute_backward -- backward of O[perm[j]] = gate[perm[j]] * Op[j]:
 *   dgate[n]    = sum over heads and channels of dO[n] * Op[j]  (n = perm[j]), float [N]
 *   dOp[j]      = gate[n] * dO[n]                               bf16 [N, H, D] (permuted)
 *   delta[h][j] = sum over channels of dOp[j, h] * Op[j, h]    float [H, N]
 *   (delta computed from the bf16-rounded dOp the attention backward reads,
 *   so that its dP - delta cancels exactly where it should).  dO bf16 [N, H, D] in
 *   original order; Op the saved attention output.  Needs no workspace.
 */
int moga_unpermute_backward(const void* dO, const void* Op, const int32_t* perm, const float* gate,
                            int64_t N, int32_t H, int32_t D, void* dOp, float* delta, float* dgate,
                            void* stream);

/*
 * moga_group_attention_backward -- gradients of the group attention (Eq. 1
 *   inside each group): with P = exp(scale Q K^T - lse) per group and head,
 *   dV = P^T dOp, dS = P * (dOp V^T - delta), dQ = scale dS K,
 *   dK = scale dS^T Q.  Inputs in permuted order (Qp, Kp, Vp, dOp bf16
 *   [N, H, D]; lse, delta float [H, N]); outputs dQ, dK, dV bf16 [N, H, D]
 *   written in ORIGINAL token order through perm (row perm[j] gets the
 *   gradient of permuted row j).  Deterministic (no atomics).
 *   ws: at least moga_workspace_bytes(MOGA_OP_ATTENTION_BACKWARD, N, M, H, D).
 *   A larger workspace lets the call keep dS in it (bf16, about n_g^2 * 2
 *   bytes per group and head) and form dQ from it: five matrix products per
 *   group and head instead of seven.  moga_attention_backward_staged_bytes()
 *   gives the size that holds every head of this call's groups; a smaller
 *   one (above 4096 bytes) holds the first Hs heads that fit, and the others
 *   are computed without dS, as with the minimum workspace.  Hs is decided on
 *   the device, from cu_seqlens; after the call the int32 at byte offset
 *   MOGA_BWD_STAGED_FLAG_OFFSET of ws reads Hs (written only when
 *   ws_bytes > 4096).  dK and dV are bitwise the same either way; dQ agrees
 *   to the float32 rounding of the product order.
 */
#define MOGA_BWD_STAGED_FLAG_OFFSET 2560
int moga_group_attention_backward(const void* Qp, const void* Kp, const void* Vp, const void* dOp,
                                  const float* lse, const float* delta, const int32_t* cu_seqlens,
                                  const int32_t* perm, int64_t N, int32_t H, int32_t D, int32_t M,
                                  float softmax_scale, void* dQ, void* dK, void* dV, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * moga_attention_backward_staged_bytes -- workspace of
 *   moga_group_attention_backward that keeps dS of all H heads for these
 *   groups: 4096 + H * sum over groups of ceil(n_g / 32) * (that rounded up
 *   to even) * 2048 bytes (each head adds an equal share).  cu_seqlens_host: HOST int32 [M + 1] (a copy of the device array).
 *   0 for invalid arguments (M outside 1..64, H < 1, a negative group size or
 *   one above 2^24 tokens).  Host-only, no device call.
 */
size_t moga_attention_backward_staged_bytes(const int32_t* cu_seqlens_host, int32_t M, int32_t H);

/*
 * moga_route_backward -- router gradients from dgate (section "MoGA Router",
 *   Eq. 3 differentiated with the hard choice held fixed): with p the softmax
 *   of the recomputed logits r = X W_r^T (+ bias) and g = group_id,
 *   dlogits[n][j] = dgate[n] * p_g * ([j == g] - p_j), then
 *   dX = dlogits W_r (float [N, d_model]), dWr = dlogits^T X (float [M, d_model]),
 *   dbias = sum_n dlogits[n] (float [M]; may be NULL).  Fixed-order
 *   reductions (bitwise repeatable).  X, Wr bf16 as moga_route; d_model a
 *   multiple of 32.  ws: moga_workspace_bytes(MOGA_OP_ROUTE_BACKWARD, N, M, 1, d_model).
 */
int moga_route_backward(const void* X, const void* Wr, const float* bias, const int32_t* group_id,
                        const float* dgate, int64_t N, int32_t d_model, int32_t M, float* dX,
                        float* dWr, float* dbias, void* ws, size_t ws_bytes, void* stream);

/*
 * moga_workspace_bytes -- bytes of workspace `op` needs for these sizes
 *   (0 when the op needs none, or when the sizes are invalid).  Host-only.
 */
size_t moga_workspace_bytes(int32_t op, int64_t N, int32_t M, int32_t H, int32_t D);

/* moga_strerror -- static description of a moga_status.  Host-only. */
const char* moga_strerror(int32_t status);

/* moga_version -- library version as major * 10000 + minor * 100 + patch. */
int32_t moga_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOGA_H_ */
