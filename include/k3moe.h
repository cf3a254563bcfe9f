/*
 * k3moe — one routed Mixture-of-Experts FFN layer on MXFP4 experts, for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the MoE block of the Kimi-K3-style model the pages describe:
 * per token, a router picks 16 of 896 routed experts, each expert is a gated
 * FFN whose weights are MXFP4 (4-bit E2M1 codes with one E8M0 scale per 32
 * weights, multiplied directly rather than expanded to a dense copy), and 2
 * always-on shared experts are added for every token (kimi-k3-in-c review
 * page, "at a glance" and "KDA/MLA/MoE" tables; translated README, "shard
 * census"; explainer page, "reduction one").  The routing rule, the gated
 * activation and the combine order taken here are:
 *   logits[t][e] = sum_i x[t][i] Wr[e][i]
 *   S_t          = k largest logits, ties to the lower expert id
 *   w[t][e]      = exp(l_e) / sum_{j in S_t} exp(l_j)     (softmax over S_t)
 *   y_(t,e)      = Wd_e (silu(Wg_e x_t) * (Wu_e x_t)),    silu(z) = z / (1 + e^-z)
 *   out[t]       = (shared_0(x_t) + shared_1(x_t) + ...)
 *                  + sum over S_t in ascending expert id, skipping w = 0, of w y
 * (the pages' own model uses sigmoid scores with a selection-only bias and a
 * bounded-tanh gate; this library implements the softmax / SiLU form).
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers unless stated; the caller
 *     allocates and owns every buffer (weights, activations, outputs,
 *     workspace, diagnostics).  The library allocates nothing, keeps no
 *     mutable global state and may run concurrently on different streams
 *     when the workspaces differ.
 *   - `stream` is a hipStream_t (NULL = the null stream).  A call validates
 *     its arguments on the host, enqueues its kernels on `stream` and returns
 *     without synchronising; buffers must stay valid until the work is done.
 *   - Validation happens before any launch: a non-OK status means nothing was
 *     enqueued (except K3MOE_EHIP, where earlier kernels of the same call may
 *     have been enqueued).  No call aborts, exits or throws.
 *   - Base pointers must be 16-byte aligned (K3MOE_EALIGN otherwise).
 *   - Results are deterministic: the same inputs give the same bits on every
 *     run, and a token's outputs do not depend on the other tokens of the
 *     batch as long as the batch stays within one path class
 *     (k3moe_path_class).
 */
#ifndef K3MOE_H
#define K3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum k3moe_status {
  K3MOE_OK = 0,
  K3MOE_EINVAL = 1,       /* NULL required pointer, negative or inconsistent sizes */
  K3MOE_ESHAPE = 2,       /* shape outside the supported set (see k3moe_shape) */
  K3MOE_EALIGN = 3,       /* a base pointer is not 16-byte aligned */
  K3MOE_EWORKSPACE = 4,   /* workspace NULL or smaller than k3moe_workspace_bytes() */
  K3MOE_EUNSUPPORTED = 5, /* dtype / weight-format combination not implemented */
  K3MOE_EHIP = 6          /* a HIP launch failed; k3moe_last_error() has the detail */
} k3moe_status;

/* Activation / output element types. */
enum { K3MOE_F32 = 0, K3MOE_BF16 = 1 };
/* Expert weight formats. */
enum { K3MOE_FMT_MXFP4 = 0, K3MOE_FMT_BF16 = 1, K3MOE_FMT_RVQ3 = 2 };
/* Operation ids for k3moe_workspace_bytes(). */
enum {
  K3MOE_OP_ROUTE = 0,
  K3MOE_OP_PERMUTE = 1,
  K3MOE_OP_EXPERT_FFN = 2,
  K3MOE_OP_SHARED_FFN = 3,
  K3MOE_OP_COMBINE = 4,
  K3MOE_OP_LAYER = 5,
  K3MOE_OP_EXPERT_GATEUP = 6
};
/* Router modes (k3moe_shape.router).
 *   SOFTMAX:      S_t = k largest logits; w = softmax of the chosen logits.
 *   SIGMOID:      the pages' K3 router (kimi-k3-in-c review page,
 *                 "KDA/MLA/MoE" table: the routing bias bends only the
 *                 selection; the combine weights come from the unbiased
 *                 sigmoid scores): S_t = k largest sigmoid(l_e) + bias_e,
 *                 w_e = sigmoid(l_e).
 *   SIGMOID_NORM: the same selection, w_e = sigmoid(l_e) / sum over S_t of
 *                 sigmoid (the pages do not say whether the weights are
 *                 renormalised; both readings are offered).
 * Ties go to the lower expert id in every mode. */
enum { K3MOE_ROUTER_SOFTMAX = 0, K3MOE_ROUTER_SIGMOID = 1, K3MOE_ROUTER_SIGMOID_NORM = 2 };
/* Activation modes of the routed experts (k3moe_shape.act).
 *   EXACT: the activations enter the products as given (the pages' engines
 *          never quantise activations: kimi-k3-in-c review page,
 *          "KDA/MLA/MoE" table; explainer page, "reduction one").
 *   MXFP4: x before gate/up and h before down are quantised to MXFP4 (OCP MX
 *          v1.0: per 32-element block, scale 2^(floor(log2 max|v|) - 2),
 *          elements rounded to the nearest E2M1 value, ties to even,
 *          saturating at 6), so both operands of the matrix-core products
 *          are MXFP4 and one pass runs at the FP4 rate.  An approximation of
 *          the layer, not the layer: its outputs follow the quantised
 *          definition, not the exact one.  Needs bf16 x, d % 512 == 0 and
 *          f % 512 == 0; the routed experts then take the grouped GEMMs at
 *          every batch size. */
enum { K3MOE_ACT_EXACT = 0, K3MOE_ACT_MXFP4 = 1 };
/* Path classes (k3moe_path_class). */
enum { K3MOE_PATH_GEMV = 0, K3MOE_PATH_MFMA = 1 };

/* Device diagnostic counters: an int32 array of K3MOE_DIAG_COUNT entries the
 * caller zeroes; calls that take `diag` add to it (NULL = not collected).
 * A non-zero BAD_EXPERT_IDS or NONFINITE_LOGITS means the call finished but
 * its results are not to be trusted. */
enum {
  K3MOE_DIAG_RECHECKED_TOKENS = 0, /* tokens whose top-k set was decided by the
                                      exact fp64 re-evaluation of near-tied logits */
  K3MOE_DIAG_NONFINITE_LOGITS = 1, /* NaN/inf router logits seen */
  K3MOE_DIAG_BAD_EXPERT_IDS = 2,   /* expert ids outside [0, E) given to permute
                                      (such pairs are dropped) */
  K3MOE_DIAG_SCORE_NEAR_TIES = 3,  /* sigmoid router: tokens whose chosen set,
                                      after the exact logit recheck, still hinges
                                      on two selection scores closer than the fp64
                                      sigmoid evaluation can order (the set could
                                      differ from another fp64 implementation's) */
  K3MOE_DIAG_COUNT = 4
};

/* Problem shape.  Supported set: 0 <= T (T = 0 is an empty batch: every call
 * returns K3MOE_OK and enqueues nothing), T * k < 2^31; 32 <= d <= 16384 and
 * d % 32 == 0; 32 <= f <= 16384 and f % 32 == 0; 1 <= k <= min(E, 64);
 * E <= 1024; 0 <= n_shared <= 8; f_shared % 32 == 0 (>= 32 when n_shared > 0);
 * x_dtype, out_dtype in {K3MOE_F32, K3MOE_BF16}; router one of
 * K3MOE_ROUTER_* (0, the softmax router, for a zero-initialised shape);
 * act one of K3MOE_ACT_* (0, exact activations, when zero-initialised);
 * routed_format K3MOE_FMT_MXFP4 (0) or K3MOE_FMT_RVQ3 (with exact activations,
 * d % 128 == 0, f % 128 == 0). */
typedef struct k3moe_shape {
  int64_t T;         /* tokens */
  int32_t d;         /* hidden size */
  int32_t f;         /* routed expert intermediate size */
  int32_t E;         /* routed experts */
  int32_t k;         /* experts chosen per token */
  int32_t n_shared;  /* always-on shared experts */
  int32_t f_shared;  /* shared expert intermediate size */
  int32_t x_dtype;   /* activations x [T][d] */
  int32_t out_dtype; /* layer output [T][d] */
  int32_t router;    /* K3MOE_ROUTER_* */
  int32_t act;       /* K3MOE_ACT_* (routed experts' activation mode) */
  int32_t routed_format; /* K3MOE_FMT_MXFP4 (0) or K3MOE_FMT_RVQ3: the routed bank's format */
} k3moe_shape;

/* A bank of experts, expert-major (each expert's bytes contiguous).
 * MXFP4 (routed experts):
 *   w13       [n][2f][d/2]  u8, packed E2M1 codes; rows 0..f-1 gate, f..2f-1 up
 *   w13_scale [n][2f][d/32] u8, E8M0 (value 2^(s-127); 255 = NaN)
 *   w2        [n][d][f/2]   u8
 *   w2_scale  [n][d][f/32]  u8
 *   Byte i of a row holds element 2i in its low nibble, 2i+1 in its high
 *   nibble; elements 32b..32b+31 share scale byte b of the row.
 * BF16 (shared experts): w13 [n][2f][d], w2 [n][d][f] bf16; scales NULL.
 * RVQ3 (routed experts, the pages' second format: residual vector
 * quantisation at 3.00 bits per weight — WASTE article page, section
 * "정확성 검증과 양자화"): every 8-weight vector is the sum of one entry of
 * each of three 256-entry codebooks of its matrix,
 *   W[r][8g + j] = C_0[i_0[r][g]][j] + C_1[i_1[r][g]][j] + C_2[i_2[r][g]][j];
 *   w13       [n][3][d/128][2f][16] u8 indices (stage, slice of 16 groups,
 *             row, group within the slice); rows 0..f-1 gate, f..2f-1 up
 *   w13_scale [n][3][256][8] fp32 codebooks C_s of w13
 *   w2        [n][3][f/128][d][16] u8, w2_scale [n][3][256][8] fp32
 *   (needs d % 128 == 0 and f % 128 == 0; shape.routed_format = RVQ3). */
typedef struct k3moe_expert_bank {
  int32_t format;    /* K3MOE_FMT_MXFP4 or K3MOE_FMT_BF16 */
  int32_t n_experts;
  int32_t d, f;
  const void* w13;
  const void* w13_scale;
  const void* w2;
  const void* w2_scale;
} k3moe_expert_bank;

typedef struct k3moe_layer_weights {
  const void* w_router;      /* [E][d] bf16 */
  k3moe_expert_bank routed;  /* MXFP4, n_experts = E, f = shape.f */
  k3moe_expert_bank shared;  /* BF16, n_experts = n_shared, f = shape.f_shared */
  const float* router_bias;  /* [E] fp32 selection bias of the sigmoid routers,
                                NULL = none; must be NULL for the softmax router */
} k3moe_layer_weights;

/* Bytes of workspace `op` needs for `shape` (0 for an invalid shape).  The
 * workspace pointer must be 256-byte aligned.  Host-only; no passage defines
 * it (the pages' engines size their buffers from the shard census, translated
 * README, "shard census"). */
size_t k3moe_workspace_bytes(const k3moe_shape* shape, int op);

/* Bytes of an MXFP4 matrix of rows x cols: rows * cols * 17 / 32 (half a byte
 * per E2M1 code plus one E8M0 byte per 32 weights — the 0.53125 bytes per
 * weight of the pages' shard census).  Host-only helper. */
uint64_t k3moe_mxfp4_bytes(int64_t rows, int64_t cols);

/* Which path class a call with this shape takes (a token's output bits
 * depend on which class its batch falls in, never on anything else about the
 * batch; within the MFMA class, on whether T is below 512 or not, see the
 * router).  The class is K3MOE_PATH_MFMA when T >= 32, x is bf16,
 * d % 512 == 0 and f % 512 == 0, and K3MOE_PATH_GEMV otherwise.
 *   - Router: fp64 GEMVs in the GEMV class; fp64 matrix-core tiles in the
 *     MFMA class below 512 tokens; from 512 tokens bf16 matrix-core logits
 *     with a bound, the experts that can still reach the top k re-evaluated
 *     in fp64.  The chosen set is the same bits every way (see k3moe_route);
 *     the weights come from fp64 logits of three arrangements, so they can
 *     differ in the last bits across these lines.
 *   - Shared experts: bf16 matrix-core GEMMs in the MFMA class when
 *     f_shared % 128 == 0; otherwise (GEMV class, or another f_shared) GEMVs
 *     with fp32 dot products, one pass over the weights per token.
 *   - Routed experts: whenever x is bf16, d % 512 == 0 and f % 512 == 0,
 *     in both classes, the scaled MXFP4 matrix-core instruction (the stored
 *     weight bytes as one operand, the activations split exactly into E4M3
 *     passes with E8M0 block scales as the other; one workgroup per active
 *     expert and output slice for one token, grouped GEMMs for more), so a
 *     token's routed outputs are the same bits at every batch size; otherwise
 *     fp32 GEMVs, the same bits at every batch size too.
 * Results of the two classes agree within the stated tolerance, not bit for
 * bit.  Returns K3MOE_PATH_GEMV for an invalid shape. */
int k3moe_path_class(const k3moe_shape* shape);

/* Router + top-k + weights.  Passage: 16 of 896 routed experts chosen per
 * token by a linear router over the hidden state (kimi-k3-in-c review page,
 * "at a glance" and "KDA/MLA/MoE" tables; translated README, "shard census");
 * shape->router picks the selection and weight rule (K3MOE_ROUTER_*: the
 * pages' sigmoid router with its selection-only bias, or the softmax router
 * of the workload definitions); the tie rule is this library's reading.
 * x [T][d] (x_dtype), w_router [E][d] bf16, router_bias [E] fp32 (sigmoid
 * routers only, NULL = no bias) ->
 *   topk_idx [T][k] int32, each row in ascending expert id;
 *   topk_w   [T][k] fp32, aligned with topk_idx (summing to 1 per token for
 *            the softmax and renormalised sigmoid routers);
 *   logits   [T][E] fp32 (optional, NULL = not written; the fp64 logits of
 *            every expert, which from 512 tokens in the MFMA class costs an
 *            extra pass of the fp64 matrix-core router).
 * The chosen set equals the set an exact evaluation of the logits in fp64
 * (ascending i) picks: near-ties at the k/k+1 boundary are re-evaluated
 * exactly on the device (counted in diag[K3MOE_DIAG_RECHECKED_TOKENS]).  For
 * the sigmoid routers the selection scores are evaluated in fp64 from those
 * logits; see K3MOE_DIAG_SCORE_NEAR_TIES for the one case left open.
 * diag: optional K3MOE_DIAG_COUNT counters (NULL = not collected); non-finite
 * logits are counted in diag[K3MOE_DIAG_NONFINITE_LOGITS].
 * Errors: EINVAL (NULL x, w_router, topk_idx, topk_w; a bias with the
 * softmax router), EUNSUPPORTED (an unknown router), EALIGN, EWORKSPACE.
 * Workspace: k3moe_workspace_bytes(shape, K3MOE_OP_ROUTE). */
k3moe_status k3moe_route(const k3moe_shape* shape, const void* x, const void* w_router,
                         const float* router_bias, int32_t* topk_idx, float* topk_w,
                         float* logits, int32_t* diag, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Counting sort of the T*k (token, slot) pairs by expert, stable in pair
 * order (pair p = t*k + slot).  Passage: the experts are gathered per layer
 * and each expert's weights are read once for all its tokens (WASTE article
 * page, section "속도는 어디서 나왔나"; explainer page, "le cache LRU"); the
 * grouping itself is this library's.  Outputs:
 *   counts [E], offsets [E+1] (exclusive prefix sum, offsets[E] = T*k),
 *   sorted_pair [T*k]: sorted_pair[q] = pair at sorted position q,
 *   pair_pos    [T*k]: its inverse.
 * Exact integer results.  An id outside [0, E), or an id repeated within a
 * token's row, is dropped (its pair_pos is -1, sorted positions past
 * offsets[E] hold -1) and counted in diag[K3MOE_DIAG_BAD_EXPERT_IDS].
 * Errors: EINVAL (a NULL output), EALIGN, EWORKSPACE.
 * Workspace: k3moe_workspace_bytes(shape, K3MOE_OP_PERMUTE). */
k3moe_status k3moe_permute(const k3moe_shape* shape, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                           int32_t* diag, void* workspace, size_t workspace_bytes, void* stream);

/* Expert FFN y = Wd (silu(Wg x) * (Wu x)).  Passage: routed experts stored
 * as MXFP4 and multiplied without a dequantised copy (kimi-k3-in-c review
 * page, "KDA/MLA/MoE" table; explainer page, "reduction one"); the gated
 * activation is taken as SiLU (the pages name a bounded "SiTU" gate without
 * a formula).
 * Routed mode (bank MXFP4 or RVQ3 as shape.routed_format says, n_experts = E;
 * sorted_pair != NULL; RVQ3 banks are multiplied through per-token
 * partial-dot tables of their codebooks, the WASTE article page's method):
 *   y [T*k][d] fp32, row q = expert e's FFN of token sorted_pair[q] / k,
 *   where e is the expert whose range offsets[e] .. offsets[e+1] holds q;
 *   unweighted.  offsets and sorted_pair as written by k3moe_permute.
 *   Workspace: k3moe_workspace_bytes(shape, K3MOE_OP_EXPERT_FFN).
 * Shared mode (bank BF16, n_experts = n_shared, f = f_shared;
 *   sorted_pair == NULL, offsets ignored): every token through every expert
 *   of the bank with weight 1, summed in bank order: y [T][d] fp32, the same
 *   call as k3moe_shared_ffn (same kernels, same bits).
 *   Workspace: k3moe_workspace_bytes(shape, K3MOE_OP_SHARED_FFN).
 * Errors: EINVAL (NULL pointers, bank not matching the shape),
 * EUNSUPPORTED (an MXFP4 bank without sorted_pair, a BF16 bank with one),
 * EALIGN, EWORKSPACE. */
k3moe_status k3moe_expert_ffn(const k3moe_shape* shape, const k3moe_expert_bank* bank,
                              const void* x, const int32_t* offsets, const int32_t* sorted_pair,
                              float* y, void* workspace, size_t workspace_bytes, void* stream);

/* The two halves of k3moe_expert_ffn's routed mode (same kernels, same
 * bits; the passage is k3moe_expert_ffn's):
 * gate/up + SiLU-GLU:  h, row q = silu(Wg x) * (Wu x) of expert e on token
 *   sorted_pair[q] / k (e as for k3moe_expert_ffn);
 * down:  y [T*k][d] fp32, row q = Wd_e h[q].
 * h is a buffer of [T*k][f] 32-bit words.  Its form follows the routed
 * experts' kernels, which take the scaled matrix-core instruction whenever x
 * is bf16, d % 512 == 0 and f % 512 == 0 (at every T, in both path classes):
 * then row q starts at byte q * (f/128) * 400 and is f/128 stages of 400
 * bytes, the value split into 3 E4M3 passes with one E8M0 scale per pass and
 * 32-feature block (h ~ sum_p code_p * 2^(scale_p - 127)): 3 x 128 code bytes
 * in feature order, then byte 4p + b = scale of pass p, block b, then 4
 * unused bytes; this is the operand form of the instruction.  With
 * act == K3MOE_ACT_MXFP4, row q starts at byte q * (f/128) * 80 and is f/128
 * stages of 80 bytes: 4 blocks of 16 E2M1 code bytes (byte i = feature 2i
 * low nibble, 2i+1 high nibble), then byte b = E8M0 scale of block b, then
 * 12 unused bytes.  Otherwise (fp32 x, or other d, f) h holds fp32 values,
 * row q at word q * f.  A buffer
 * written by k3moe_expert_gateup is meant for k3moe_expert_down with the same
 * shape.
 * Workspace (gate/up only): k3moe_workspace_bytes(shape, K3MOE_OP_EXPERT_GATEUP)
 * (0 for the fp32 form, where NULL is accepted): x in E4M3 passes. */
k3moe_status k3moe_expert_gateup(const k3moe_shape* shape, const k3moe_expert_bank* bank,
                                 const void* x, const int32_t* offsets,
                                 const int32_t* sorted_pair, float* h, void* workspace,
                                 size_t workspace_bytes, void* stream);
/* (k3moe_expert_down takes MXFP4 banks only: the RVQ3 down product keeps its
 * slice partial sums in a workspace, which k3moe_expert_ffn provides.) */
k3moe_status k3moe_expert_down(const k3moe_shape* shape, const k3moe_expert_bank* bank,
                               const float* h, const int32_t* offsets, float* y, void* stream);

/* Shared experts on a BF16 bank (n_experts = n_shared, f = f_shared):
 *   y [T][d] fp32 = sum over the bank's experts in order of each expert's FFN.
 * Passage: 2 always-on shared experts beside the routed ones, resident and
 * never streamed (kimi-k3-in-c review page, "at a glance" table and the
 * memory discussion; translated README, "shard census").  Equivalent to
 * k3moe_expert_ffn's shared mode.  Errors: EINVAL (no shared experts, NULL
 * pointers), EUNSUPPORTED (bank not BF16), EALIGN, EWORKSPACE.
 * Workspace: k3moe_workspace_bytes(shape, K3MOE_OP_SHARED_FFN). */
k3moe_status k3moe_shared_ffn(const k3moe_shape* shape, const k3moe_expert_bank* bank,
                              const void* x, float* y, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Fixed-order combine.  Passage: a fixed summation order pins the bits of
 * the pages' engine (translated README, "why no BLAS"); the order itself
 * (shared experts first, then the routed ones by ascending id, weight-0
 * terms skipped) is this library's reading.  Errors: EINVAL (NULL y_perm,
 * pair_pos, topk_w, out), EALIGN.
 *   out[t][o] = shared_y[t][o] (0 when shared_y is NULL)
 *               + sum over slots s ascending with topk_w[t][s] != 0 of
 *                 topk_w[t][s] * y_perm[pair_pos[t*k+s]][o]
 * y_perm [T*k][d] fp32, pair_pos [T*k], topk_w [T][k] fp32,
 * out [T][d] in out_dtype (bf16 by round-to-nearest-even). */
k3moe_status k3moe_combine(const k3moe_shape* shape, const float* y_perm, const int32_t* pair_pos,
                           const float* topk_w, const float* shared_y, void* out, void* stream);

/* The whole layer: route, permute, routed experts, shared experts, combine.
 * Passage: one MoE FFN layer of the pages' model (kimi-k3-in-c review page,
 * "at a glance" and "KDA/MLA/MoE" tables).
 * Bit-identical to calling the five stages above in sequence on the same
 * stream.  out [T][d] in out_dtype.  diag as for k3moe_route and
 * k3moe_permute (NULL = not collected).  Errors: those of the stages.
 * Workspace: k3moe_workspace_bytes(shape, K3MOE_OP_LAYER). */
k3moe_status k3moe_layer(const k3moe_shape* shape, const k3moe_layer_weights* weights,
                         const void* x, void* out, int32_t* diag, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Bytes of the fixed device scratch buffer of k3moe_layer_noalloc. */
#define K3MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* The whole layer without allocating and without a workspace argument, for
 * callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, hosts that forbid allocation).  Same kernels and same
 * bits as k3moe_layer; the workspace is a fixed device array of
 * K3MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends (its address is looked up once per device, on the
 * first call made with that device current).
 * Limits: the call's k3moe_workspace_bytes(shape, K3MOE_OP_LAYER) must fit
 * the buffer (K3MOE_EWORKSPACE otherwise, nothing enqueued); at d = 7168,
 * f = 2048, 896 experts top-16 that is up to 103 tokens.
 * Every call on one GPU shares that GPU's buffer: calls that may overlap on
 * one GPU (other streams, other threads) race and must not be issued.
 * Nothing in the buffer has to start at zero.  Errors: those of
 * k3moe_layer, K3MOE_EWORKSPACE as above, K3MOE_EHIP if the buffer's address
 * cannot be looked up. */
k3moe_status k3moe_layer_noalloc(const k3moe_shape* shape, const k3moe_layer_weights* weights,
                                 const void* x, void* out, int32_t* diag, void* stream);

/* ---------------------------------------------------------------------------
 * Host-resident routed experts streamed into an HBM expert cache.  Passage:
 * the pages' engines keep the routed experts out of fast memory and the hot
 * ones in an LRU cache whose size is a dial with the same outputs at every
 * budget (kimi-k3-in-c review page, "at a glance" list and memory ladder;
 * explainer page, "le cache LRU"); WASTE overlaps expert reads with compute
 * and prefetches with a router run one layer early (WASTE article page,
 * section "속도는 어디서 나왔나").  Here the experts sit in pinned host
 * memory, the cache is a bank of `slots` experts in HBM (caller-owned, MXFP4
 * layout with n_experts = slots), and misses travel over PCIe on a copy
 * stream while the shared experts run.  Outputs are the same bits as
 * k3moe_layer's on a resident bank, at every cache size.
 * The cache object is host state created by the library (the only host
 * allocation it makes); one call at a time uses a cache (calls on one cache
 * from several threads are serialised).
 * ------------------------------------------------------------------------- */
typedef struct k3moe_expert_cache k3moe_expert_cache;
typedef struct k3moe_cache_stats {
  int64_t lookups;        /* one per distinct expert of a batch (prefetches are not lookups) */
  int64_t hits;           /* lookups found resident */
  int64_t misses;         /* lookups copied in */
  int64_t prefetched;     /* experts copied in by k3moe_cache_prefetch */
  int64_t prefetch_hits;  /* hits on an expert a prefetch brought in */
  int64_t evictions;      /* resident experts replaced */
  int64_t bytes_copied;   /* host-to-device bytes (including planned-only copies) */
} k3moe_cache_stats;

/* Creates a cache for `shape` (T ignored; MXFP4 routed experts, exact
 * activations) over host_bank (HOST pointers to pinned memory, n_experts = E,
 * caller-owned) and slot_bank (DEVICE pointers, n_experts = slots with
 * k <= slots <= 1024, caller-owned; its contents are the cache's).  No GPU
 * work.  Errors: EINVAL, ESHAPE, EALIGN, EUNSUPPORTED (not MXFP4). */
k3moe_status k3moe_cache_create(const k3moe_shape* shape, const k3moe_expert_bank* host_bank,
                                const k3moe_expert_bank* slot_bank, k3moe_expert_cache** cache);
void k3moe_cache_destroy(k3moe_expert_cache* cache);
/* Workspace of k3moe_cache_layer for `shape` and `slots` (0 if invalid). */
size_t k3moe_cache_workspace_bytes(const k3moe_shape* shape, int32_t slots);
/* The whole layer with the routed experts taken through the cache: routes on
 * `stream`, synchronises `stream` once to read the expert ids, makes every
 * distinct expert resident (hits refresh their slot; misses replace the
 * least recently used slot this batch does not need, copied on copy_stream,
 * or on `stream` when copy_stream is NULL), runs the shared experts while
 * the copies fly, then the routed experts on slot ids and the combine.
 * A slot is refilled only after the kernels of the previous layer call and
 * the copies enqueued before have finished with it, whatever the streams
 * (events; the host also waits for the previous call's kernels before it
 * plans).  weights->routed is ignored (the cache's banks serve instead).
 * Errors: those
 * of k3moe_layer; K3MOE_ESHAPE when the batch routes to more distinct experts
 * than there are slots (the route kernels have run then, nothing else). */
k3moe_status k3moe_cache_layer(k3moe_expert_cache* cache, const k3moe_shape* shape,
                               const k3moe_layer_weights* weights, const void* x, void* out,
                               int32_t* diag, void* workspace, size_t workspace_bytes,
                               void* stream, void* copy_stream);
/* Brings the experts `ids` (HOST array) in ahead of use, copies on
 * copy_stream: the lookahead of the pages (the caller predicts, for example
 * with a router run early; the routing itself still decides).  The copies
 * wait on the GPU for the last layer call's kernels; the host does not wait.
 * Stops early, without error, when every slot is taken by this prefetch. */
k3moe_status k3moe_cache_prefetch(k3moe_expert_cache* cache, const int32_t* ids, int32_t n,
                                  void* copy_stream);
/* Host-only planning, no copies and no GPU work: makes the distinct experts
 * `ids` resident as one batch would and writes their slots (for tests of the
 * replacement policy).  Errors: EINVAL, ESHAPE (more ids than slots). */
k3moe_status k3moe_cache_plan(k3moe_expert_cache* cache, const int32_t* ids, int32_t n,
                              int32_t* slot_of);
/* Counters since creation. */
k3moe_status k3moe_cache_stats_get(const k3moe_expert_cache* cache, k3moe_cache_stats* stats);

/* Static description of a status code. */
const char* k3moe_status_str(k3moe_status status);
/* Detail of the last non-OK status returned on the calling thread. */
const char* k3moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* K3MOE_H */
