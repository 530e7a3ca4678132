/*
 * moe_mi355x.h -- C ABI of the sparsely-gated Mixture-of-Experts layer forward
 * on one AMD Instinct MI355X (gfx950).
 *
 * The layer (web page "Mixture of Experts: Scaling Parameters Without Scaling
 * Compute", section "The MoE layer"): for each token x the router computes
 * logits g = W_r x and probabilities p = softmax(g), keeps the top-k experts,
 * optionally renormalises their probabilities, runs each chosen expert
 * FFN_e(x) = W2_e GELU(W1_e x + b1_e) + b2_e and returns the probability-
 * weighted sum of their outputs.  The layer also returns the Switch-style
 * auxiliary loss aux = E * sum_i f_i P_i (same page, section "The central
 * problem: load balancing").  An optional expert capacity C limits every
 * expert to C assignments, taken in token order (same section; also "Experts
 * also have capacity limits" on the llmdaily day-59 page); the overflow is
 * either dropped or rerouted to the token's next-best experts (moe_desc.
 * capacity_policy).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer (HIP device memory, or
 * memory the device can address) unless it says otherwise; descriptors are
 * HOST pointers.  All device pointers must be 16-byte aligned.  Layouts are
 * row-major; weights use the [out][in] layout of a linear layer.
 * Ownership.  The caller allocates and frees every buffer, including the
 * workspace sized by moe_workspace_size().  The library never allocates or
 * frees device memory, never synchronises the stream or the device, and
 * keeps no state between calls except a thread-local error message.
 * Aliasing.  No output, the workspace included, may overlap another output or
 * an input of the same call (byte ranges from the descriptor's shapes); a call
 * that finds such an overlap returns MOE_ERR_INVALID.  moe_route's topk_idx
 * counts as an output.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Every call only enqueues work on that stream, in order; buffers
 * must stay alive until the stream has passed that work.
 * Errors.  Every call validates its arguments on the host first; on any
 * status other than MOE_OK nothing has been enqueued, and moe_last_error()
 * describes the problem.  A failed kernel launch returns MOE_ERR_HIP; faults
 * inside kernels surface when the caller synchronises.  No C++ exception
 * crosses this interface.
 * Precision.  x, the weights and the expert biases share `dtype`.  Matrix
 * products accumulate in fp32; router logits, probabilities, the routing
 * weights, the expert outputs `o` and the layer output `y` are fp32.  With
 * dtype BF16 the post-GELU activations `h` are stored as moe_desc.h_mode says
 * (rounded to bf16, nearest-even, or kept as two bf16 terms).
 * Determinism.  No call uses floating-point atomics; repeated calls on the
 * same inputs give bitwise-identical results.
 * Limits.  1 <= tokens; 1 <= n_experts <= 64; 1 <= top_k <= min(8, n_experts);
 * d_model, d_ff and d_ff_shared are multiples of 128; tokens * top_k *
 * max(d_model, d_ff) and tokens * d_ff_shared must fit in int32, and one
 * expert's weight matrix (d_model x max(d_ff, d_ff_shared) elements) must be
 * under 4 GiB (else MOE_ERR_UNSUPPORTED).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,      /* bad argument: shape, option, null or misaligned pointer */
  MOE_ERR_UNSUPPORTED = -2,  /* valid layer, outside what this library implements */
  MOE_ERR_WORKSPACE = -3,    /* workspace pointer NULL or smaller than moe_workspace_size() */
  MOE_ERR_HIP = -4           /* the HIP runtime refused a launch */
};

/* Expert-FFN kernel choice (moe_desc.ffn_path).  Averages are the host's bound,
 * min(T*k, E*C) / E rows per expert.  AUTO resolves to TILED (LDS-tiled, bf16
 * only) for bf16 layers averaging >= 64 rows per expert, with 256-row tiles from
 * 256 rows per expert (MFMA-bound prefill) and 128-row tiles below; and to
 * STREAM (weight-streaming, HBM-bound) otherwise. */
enum { MOE_FFN_AUTO = 0, MOE_FFN_TILED = 1, MOE_FFN_STREAM = 2 };

/* Storage of the post-GELU activations h for a bf16 layer (moe_desc.h_mode).
 *   MOE_H_BF16:  h rounded to bf16, [T*k][F] bf16 (2 bytes per element).
 *   MOE_H_SPLIT: h kept as two bf16 terms, h = hi + lo with hi = bf16(h) and
 *                lo = bf16(h - hi): plane hi [T*k][F] followed by plane lo
 *                [T*k][F] (4 bytes per element in total); the second product
 *                runs one MFMA per term, so o carries ~16 bits of h.
 *   MOE_H_AUTO:  BF16 on the TILED path at >= 256 rows per expert (MFMA-bound),
 *                SPLIT below that and on the STREAM path, where the products
 *                are weight-bound and the second term costs little, and SPLIT
 *                for top-1 layers without renormalisation (below).
 * For an fp32 layer h is fp32 [T*k][F] and h_mode must be AUTO.  On the TILED
 * path SPLIT uses 128-row tiles.
 * MOE_H_BF16 on a top-1 layer without renormalisation returns
 * MOE_ERR_UNSUPPORTED: there y_t = p_t * FFN(x_t) with the raw probability p_t,
 * and capacity drops add zero rows, so max|y - y_exact| / RMS(y) is far larger
 * than for averaged outputs; with bf16-rounded h it measured 0.025 (777
 * tokens, 64 experts, capacity 16) and 0.041 (8192 tokens, 64 experts,
 * capacity 160), past the 2e-2 bar, while two bf16 terms keep it near 1e-5. */
enum { MOE_H_AUTO = 0, MOE_H_BF16 = 1, MOE_H_SPLIT = 2 };

/* What happens to assignments past an expert's capacity (moe_desc.capacity_policy).
 *   MOE_CAPACITY_DROP:    the first C assignments of each expert in token order are
 *                         kept, the rest dropped (moe_permute applies it).
 *   MOE_CAPACITY_REROUTE: rounds (moe_route applies it).  Round 0 asks every slot's
 *                         router choice.  In a round each expert accepts the requests
 *                         in token order while it has capacity left; a rejected slot
 *                         asks, in the next round, for its token's best-ranked expert
 *                         the token has not asked yet (ranked as the top-k is; a
 *                         token's rejected slots take these in slot order); a slot
 *                         with no expert left is dropped.  A served slot's weight is
 *                         the probability of the expert serving it over the original
 *                         denominator (the sum of the k chosen probabilities when
 *                         renormalising, else 1).  Needs capacity > 0. */
enum { MOE_CAPACITY_DROP = 0, MOE_CAPACITY_REROUTE = 1 };

/* Options of one layer call (host struct). */
typedef struct moe_desc {
  int32_t tokens;          /* T */
  int32_t d_model;         /* d */
  int32_t d_ff;            /* F, hidden width of every expert */
  int32_t n_experts;       /* E */
  int32_t top_k;           /* k */
  int32_t renormalize;     /* 1: divide the chosen probabilities by their sum */
  int32_t capacity;        /* C > 0: at most C assignments per expert; 0: no limit */
  int32_t dtype;           /* MOE_DTYPE_* */
  int32_t has_expert_bias; /* 1: b1 and b2 are given; 0: both absent */
  int32_t ffn_path;        /* MOE_FFN_*: AUTO picks by rows per expert; the others force a kernel */
  int32_t h_mode;          /* MOE_H_*: storage of the post-GELU activations h */
  int32_t d_ff_shared;     /* Fs: hidden width of the shared expert, a multiple of 128; 0 = none.
                              The shared expert (web page "Mixture of Experts: Scaling Parameters
                              Without Scaling Compute", section "Design variations": shared
                              experts, always active) runs on every token and its output is added
                              to y with weight 1.  Several shared experts are one of their joint
                              width: W1s stacked along the hidden axis, W2s side by side, b2s
                              summed. */
  int32_t capacity_policy; /* MOE_CAPACITY_*: overflow past the capacity is dropped or rerouted */
} moe_desc;

/* What the library will run for a descriptor (host struct, filled by moe_query_plan). */
typedef struct moe_plan {
  int32_t ffn_path;        /* resolved MOE_FFN_TILED or MOE_FFN_STREAM */
  int32_t h_mode;          /* resolved MOE_H_BF16 or MOE_H_SPLIT (MOE_H_AUTO for fp32 layers) */
  size_t h_bytes;          /* bytes of the h buffer moe_ffn_up writes: T*k*F*(2 or 4) */
  size_t workspace_bytes;  /* same value as moe_workspace_size() */
} moe_plan;

/* Layer parameters (device pointers). */
typedef struct moe_weights {
  const void* w_router;    /* [E][d]    dtype  (router has no bias on the pages) */
  const float* b_router;   /* [E]       fp32 logit bias added before softmax, or NULL */
  const void* w1;          /* [E][F][d] dtype */
  const void* b1;          /* [E][F]    dtype, NULL iff !has_expert_bias */
  const void* w2;          /* [E][d][F] dtype */
  const void* b2;          /* [E][d]    dtype, NULL iff !has_expert_bias */
  const float* b_select;   /* [E]       fp32 selection-only bias, or NULL: experts are ranked by
                              logit + b_select, the routing weights stay softmax(logits)
                              (web page "Mixture of Experts: Scaling Parameters Without Scaling
                              Compute", section "The central problem: load balancing",
                              auxiliary-loss-free balancing) */
  const void* w1_shared;   /* [Fs][d] dtype, NULL iff d_ff_shared == 0 */
  const void* b1_shared;   /* [Fs]    dtype, NULL iff d_ff_shared == 0 or !has_expert_bias */
  const void* w2_shared;   /* [d][Fs] dtype, NULL iff d_ff_shared == 0 */
  const void* b2_shared;   /* [d]     dtype, NULL iff d_ff_shared == 0 or !has_expert_bias */
} moe_weights;

/* Routing results (device pointers).  Which fields a call reads or writes is
 * stated at each call; in moe_forward any field may be NULL (the workspace is
 * used instead). */
typedef struct moe_routing {
  int32_t* topk_idx;       /* [T][k] chosen experts in rank order: logit descending, ties -> lower index.
                              With MOE_CAPACITY_REROUTE: the expert serving each slot, -1 if dropped */
  float* topk_w;           /* [T][k] routing weights: probabilities, renormalised over the k if asked.
                              With MOE_CAPACITY_REROUTE: the serving expert's weight, 0 if dropped */
  int32_t* counts;         /* [E]    rows kept per expert (after capacity) */
  int32_t* offsets;        /* [E+1]  exclusive prefix sum of counts; offsets[E] = R, total kept rows */
  int32_t* dest;           /* [T][k] row of assignment (t,s) in x_perm/h/o, -1 if dropped */
  int32_t* src;            /* [T*k]  rows < R hold the assignment id t*k+s; rows >= R are not written */
  int32_t* top1_count;     /* [E]    tokens whose first choice is e, before capacity (defines f_e) */
  float* prob_mean;        /* [E]    P_e = mean over tokens of p_e */
  float* z_loss;           /* [1]    router z-loss: mean over tokens of (log sum_e exp logit_e)^2
                              (same page and section, router z-loss); logits include b_router,
                              not b_select */
  int32_t* reroute_rounds; /* [1]    acceptance rounds the reroute policy ran (0 without it) */
} moe_routing;

/* Status code -> static string. */
const char* moe_status_string(int status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* moe_last_error(void);

/* Bytes of workspace that any call below needs for this descriptor (host
 * output).  One workspace of this size serves every entry point. */
int moe_workspace_size(const moe_desc* desc, size_t* bytes);

/* Resolve the descriptor's AUTO choices (host output). */
int moe_query_plan(const moe_desc* desc, moe_plan* plan);

/* Router (web page "Mixture of Experts: Scaling Parameters Without Scaling
 * Compute", section "The MoE layer", steps 1-2: logits, softmax, top-k, renormalised
 * weights; section "The central problem: load balancing": the aux loss, the
 * router z-loss and the selection-only bias; llmdaily day-59 page, section
 * "Replace one MLP with many experts": the eight-expert routing example).
 * Router: logits = x W_r^T (+ b_router), softmax, top-k by logit (+ b_select
 * when given), routing weights, the aux loss and the router z-loss; with
 * MOE_CAPACITY_REROUTE also the rerouting of the overflow (one extra
 * single-workgroup kernel).
 *   x [T][d] dtype.  Writes out->topk_idx and out->topk_w (both required),
 *   out->top1_count, out->prob_mean, out->z_loss and out->reroute_rounds (each
 *   optional), and *aux (device fp32 scalar, optional):
 *   aux = E * sum_e (top1_count_e / T) * P_e, from the router's own choices. */
int moe_route(const moe_desc* desc, const void* x, const moe_weights* w, moe_routing* out,
              float* aux, void* workspace, size_t workspace_bytes, void* stream);

/* Dispatch (web page "Mixture of Experts: Scaling Parameters Without Scaling
 * Compute", section "The MoE layer": each expert processes the tokens routed to
 * it; section "The central problem: load balancing": expert capacity, overflow
 * dropped; llmdaily day-59 page, section "Experts also have capacity limits").
 * Dispatch: per-expert histogram of the assignments, prefix scan, capacity
 * (MOE_CAPACITY_DROP), stable ranks in token order, and the gather of token
 * rows into expert-contiguous rows.
 *   Reads r->topk_idx; ids outside [0, E) are dropped assignments.  Writes r->counts, r->offsets, r->dest, r->src (all
 *   required) and x_perm [T*k][d] dtype: rows 0..R-1 get x_perm[dest[t][s]] = x[t];
 *   rows >= R are not written.  Inside expert e's segment rows follow token order. */
int moe_permute(const moe_desc* desc, const void* x, moe_routing* r, void* x_perm,
                void* workspace, size_t workspace_bytes, void* stream);

/* First expert product (web page "Mixture of Experts: Scaling Parameters
 * Without Scaling Compute", section "The MoE layer": each expert is
 * Linear(d -> d_ff), GELU, Linear(d_ff -> d); this is the first linear map and
 * the GELU, erf form).
 * First expert product with GELU fused into its epilogue:
 *   h[r] = GELU_erf(x_perm[r] W1_e^T + b1_e) for every row r of expert e's segment
 *   [offsets[e], offsets[e+1]).  x_perm [T*k][d] dtype; h is stored as the
 *   resolved h_mode says (plan.h_bytes bytes).  offsets is the device array
 *   from moe_permute. */
int moe_ffn_up(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
               const moe_weights* w, void* h, void* workspace, size_t workspace_bytes,
               void* stream);

/* The first expert product as moe_forward runs it (same page and section as
 * moe_ffn_up): no x_perm is materialised; dispatched row r reads token
 * src[r] / top_k of x straight from x [T][d] dtype.  src [T*k] and offsets
 * [E+1] are moe_permute's outputs; h as moe_ffn_up writes it, bitwise equal to
 * moe_ffn_up on the gathered rows. */
int moe_ffn_up_gather(const moe_desc* desc, const void* x, const int32_t* src,
                      const int32_t* offsets, const moe_weights* w, void* h, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Second expert product (same page and section: the expert's second linear
 * map, Linear(d_ff -> d) with its bias).
 * Second expert product: o[r] = h[r] W2_e^T + b2_e, h as moe_ffn_up wrote it,
 * o [T*k][d] fp32. */
int moe_ffn_down(const moe_desc* desc, const void* h, const int32_t* offsets,
                 const moe_weights* w, float* o, void* workspace, size_t workspace_bytes,
                 void* stream);

/* The grouped expert FFN (same page and section: every chosen expert's
 * Linear-GELU-Linear on its own rows): moe_ffn_up then moe_ffn_down on the same
 * stream. */
int moe_grouped_ffn(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                    const moe_weights* w, void* h, float* o, void* workspace,
                    size_t workspace_bytes, void* stream);

/* The shared expert (web page "Mixture of Experts: Scaling Parameters Without
 * Scaling Compute", section "Design variations": shared experts are always
 * active), on every token (desc->d_ff_shared > 0):
 *   o_shared[t] = W2s GELU(W1s x[t] + b1s) + b2s.  x [T][d] dtype, o_shared [T][d]
 *   fp32.  Its hidden activations live in the workspace. */
int moe_shared_ffn(const moe_desc* desc, const void* x, const moe_weights* w, float* o_shared,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Combine (web page "Mixture of Experts: Scaling Parameters Without Scaling
 * Compute", section "The MoE layer", step 3): y[t] = sum over slots s = 0..k-1
 * with dest[t][s] >= 0 of topk_w[t][s] * o[dest[t][s]], accumulated in fp32
 * in slot order (no atomics), plus o_shared[t] when o_shared is not NULL;
 * without a shared expert y[t] = 0 when every slot was dropped.
 *   o [T*k][d] fp32, dest [T][k], topk_w [T][k] fp32, o_shared [T][d] fp32 or
 *   NULL, y [T][d] fp32. */
int moe_combine(const moe_desc* desc, const float* o, const int32_t* dest, const float* topk_w,
                const float* o_shared, float* y, void* stream);

/* The whole layer (web page "Mixture of Experts: Scaling Parameters Without
 * Scaling Compute", section "The MoE layer": the module's forward maps x to the
 * weighted sum of the chosen experts' outputs and returns the aux loss beside
 * it; llmdaily day-59 page, section "Replace one MLP with many experts").
 * The whole layer: route, permute, grouped FFN, the shared expert (if any),
 * combine.  The first expert product reads each dispatched row's token
 * straight from x (through src), so no x_perm is materialised.
 *   x [T][d] dtype -> y [T][d] fp32 and *aux (device fp32 scalar, optional).
 *   routing may be NULL; any non-NULL field of it receives that result. */
int moe_forward(const moe_desc* desc, const void* x, const moe_weights* w, float* y, float* aux,
                moe_routing* routing, void* workspace, size_t workspace_bytes, void* stream);

/* Measurement aid, not part of the layer: one plain streaming read of `bytes`
 * bytes of device memory at buf (each wave reads its own contiguous 16 KiB),
 * the practical HBM read ceiling that the weight-bound kernels are compared
 * with.  bytes must be a positive multiple of 65536 (else MOE_ERR_INVALID);
 * sink is a device uint32 the kernel may write (never read back). */
int moe_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The call allocates nothing: it runs moe_forward on a
 * 32 MiB device array the library holds on each GPU it runs on until the
 * process ends (enough for a decode batch of a Mixtral-shaped layer: 32
 * tokens of d_model 4096, d_ff 14336, 8 experts, top-2 need 8.5 MiB).
 * Layers whose moe_workspace_size() exceeds 32 MiB return MOE_ERR_UNSUPPORTED
 * before anything is enqueued.  Arguments, results and errors are those of
 * moe_forward.  Every call on one GPU uses the same array, which keeps the
 * last call's contents: calls that overlap on one GPU (two streams, two
 * threads) race on it and must be serialised by the caller. */
int moe_forward_noalloc(const moe_desc* desc, const void* x, const moe_weights* w, float* y,
                        float* aux, moe_routing* routing, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
