/*
 * inkling_moe.h -- C ABI of the MI355X (gfx950) Inkling MoE feed-forward.
 *
 * The operation is the MoE feed-forward of the Inkling layers page
 * (nemo_automodel.components.models.inkling.layers):
 *
 *   InklingGate        logits z = x . bank^T over a gate bank of n_routed routed
 *                      rows followed by n_shared shared rows, fp32 operands;
 *                      experts selected by top_k of sigmoid(z) + correction
 *                      bias (InklingCorrectionBias); weights = softmax of
 *                      log-sigmoid over [selected routed logits || shared
 *                      logits] times route_scale * global_scale.
 *   inkling_swiglu     SwiGLU on the interleaved [g0, u0, g1, u1, ...] gate_up
 *                      output, the activated output scaled by the routing weight.
 *   InklingSharedExperts  always-on experts weighted by the shared gammas.
 *   InklingMoE.forward routed + shared outputs summed; output shaped like the
 *                      input; masked (padded) tokens get no routed rows.
 *
 * Readings where the page is silent: equal selection scores go to the lower
 * expert index and topk_* are ordered by descending score; route_scale *
 * global_scale also scales the shared gammas; silu(gate) * up without clamp;
 * padded tokens still pass through the shared experts.
 *
 * Conventions
 *   - Every tensor pointer is a DEVICE pointer to a contiguous row-major buffer
 *     owned by the caller.  The library keeps no pointer after a call returns.
 *   - dtype applies to x and the expert weights (INKLING_F32 or INKLING_BF16);
 *     out_dtype to the output (the input's dtype is the layer's own choice;
 *     INKLING_F32 returns the fp32 sum before its final rounding, and a bf16
 *     output is exactly that sum rounded to nearest-even).  The gate bank and
 *     correction bias are always fp32; routing outputs are int32 / fp32.
 *   - Weight layouts are nn.Linear [out, in]:
 *       routed_gate_up [n_routed][2*I][hidden]  row 2j = gate_j, 2j+1 = up_j
 *       routed_down    [n_routed][hidden][I]
 *       shared_gate_up [n_shared][2*I][hidden]  (NULL iff n_shared == 0)
 *       shared_down    [n_shared][hidden][I]
 *   - The caller flattens leading dimensions of the hidden states to T rows.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and is asynchronous.  No call allocates or frees device memory or
 *     synchronises.  Scratch lives in the caller's workspace, except for
 *     inkling_moe_forward_noalloc, whose scratch is a static device array that
 *     comes with the library's code on each GPU.  Calls that share a workspace
 *     must be ordered on one stream.
 *   - Arguments are checked on the host before anything is launched; an error
 *     return means nothing was enqueued (except INKLING_ERR_HIP, which reports
 *     a failed launch).
 *
 * Limits (INKLING_ERR_UNSUPPORTED otherwise): hidden % 64 == 0,
 * intermediate % 64 == 0, 1 <= top_k <= min(n_routed, 32), n_routed <= 512,
 * n_routed + n_shared <= 512, n_shared <= 16, T * top_k <= 2^31 - 257.
 */
#ifndef INKLING_MOE_H
#define INKLING_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define INKLING_OK 0
#define INKLING_ERR_INVALID_ARGUMENT (-1) /* null required pointer, negative size, top_k > n_routed, ... */
#define INKLING_ERR_UNSUPPORTED (-2)      /* dtype or size outside the limits above */
#define INKLING_ERR_WORKSPACE (-3)        /* workspace NULL or smaller than inkling_moe_workspace_size() */
#define INKLING_ERR_HIP (-4)              /* a HIP launch failed; see inkling_moe_last_hip_error() */
#define INKLING_ERR_TOO_LARGE (-5)        /* sizes need more scratch than inkling_moe_forward_noalloc holds */

typedef enum { INKLING_F32 = 0, INKLING_BF16 = 1 } inkling_dtype_t;

/* Sizes of one call.  T may be 0 (a successful no-op). */
typedef struct {
    int64_t T;            /* tokens (rows of x)                                 */
    int32_t hidden;       /* H: model width                                     */
    int32_t n_routed;     /* E: routed experts (InklingGate.num_experts)        */
    int32_t top_k;        /* k: experts per token (num_experts_per_tok)         */
    int32_t n_shared;     /* S: always-on shared experts (may be 0)             */
    int32_t intermediate; /* I: expert intermediate size (moe_intermediate_size)*/
    int32_t dtype;        /* inkling_dtype_t of x and the expert weights         */
    int32_t out_dtype;    /* inkling_dtype_t of out (the layer output): usually  */
                          /* dtype; INKLING_F32 keeps the fp32 sum unrounded     */
} inkling_moe_dims_t;

/* InklingGate parameters. */
typedef struct {
    const float* gate_bank;       /* [n_routed + n_shared][hidden] fp32: routed rows, then shared rows */
    const float* correction_bias; /* [n_routed] fp32 e_score_correction_bias                           */
    float route_scale;            /* InklingGate.route_scale                                           */
    float global_scale;           /* InklingGate.global_scale                                          */
} inkling_gate_t;

/* Expert weights (layouts above). */
typedef struct {
    const void* routed_gate_up;
    const void* routed_down;
    const void* shared_gate_up;
    const void* shared_down;
} inkling_experts_t;

/*
 * Routing outputs (InklingGate.forward returns topk_weights, topk_indices and
 * shared_gammas).  In inkling_moe_route the first three are required; in
 * inkling_moe_forward the whole struct pointer may be NULL and any member may be
 * NULL (then it is kept in the workspace only).
 *   topk_indices  [T][top_k] int32: selected experts, descending biased score,
 *                 equal scores -> lower index first.
 *   topk_weights  [T][top_k] fp32: gammas of the selected routed experts.
 *   shared_gammas [T][n_shared] fp32.
 *   expert_counts [n_routed] int32: routed (token, choice) pairs per expert,
 *                 padded tokens excluded.
 *   expert_offsets[n_routed + 1] int32: exclusive prefix sum of the counts.
 *   sorted_slots  [T * top_k] int32: slots t*top_k + i grouped by expert
 *                 (expert 0 first), ascending within an expert; only the first
 *                 expert_offsets[n_routed] entries are written.
 */
typedef struct {
    int32_t* topk_indices;
    float* topk_weights;
    float* shared_gammas;
    int32_t* expert_counts;
    int32_t* expert_offsets;
    int32_t* sorted_slots;
} inkling_route_out_t;

/* Bytes of device workspace that inkling_moe_route / inkling_moe_forward need
 * for these sizes (256-byte aligned base expected).  Returns INKLING_OK and
 * writes *bytes, or an error code for invalid / unsupported sizes. */
int inkling_moe_workspace_size(const inkling_moe_dims_t* dims, size_t* bytes);

/* InklingGate.forward plus the expert-sorted permutation.
 *   x             [T][hidden] in dims->dtype.
 *   padding_mask  [T] uint8, nonzero = padded token (excluded from the counts,
 *                 offsets and sorted slots; its topk_* entries are still
 *                 written), or NULL.                                          */
int inkling_moe_route(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                      const uint8_t* padding_mask, inkling_route_out_t* route_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* InklingMoE.forward: out[T][hidden] (dims->out_dtype) = sum over the selected
 * routed experts and all shared experts of gamma * expert(x).  out must not
 * alias x.  padding_mask as above (padded tokens get the shared experts only).
 * route_out may be NULL.
 * Precision: products accumulate in fp32; the expert outputs are summed in
 * fp32 in a fixed order and rounded once, so the result is bit-reproducible.
 * With dtype INKLING_BF16 the activation between an expert's two projections,
 * gamma * silu(gate) * up, is rounded to fp16 (nearest even), the bf16 down
 * weights are taken as fp16, which is exact for 2^-17 <= |w| < 2^16, and each
 * routed expert's output row is rounded to fp16 before the fp32 sum; both
 * intermediates must stay below 65504 in magnitude (above it they are inf). */
int inkling_moe_forward(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                        const inkling_experts_t* experts, const uint8_t* padding_mask, void* out,
                        inkling_route_out_t* route_out, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * inkling_moe_forward without the workspace argument, bit for bit the same
 * results.  Its scratch is a static device array of
 * INKLING_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held from the
 * library's load on that GPU until the process ends; the call allocates and
 * frees nothing.  Returns INKLING_ERR_TOO_LARGE, before anything is enqueued,
 * when inkling_moe_workspace_size() for these dims exceeds that size (at
 * hidden 6144, top-8, 2 shared experts, intermediate 2048 that is above 371
 * tokens; decode batches of 32 tokens need 5.8 MB).  Every call on one GPU
 * uses that GPU's one array, and the array keeps what the last call left
 * there: calls that overlap in time on one GPU (other streams, other threads)
 * race and must be ordered on one stream.  The device is the calling thread's
 * current HIP device.
 */
#define INKLING_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int inkling_moe_forward_noalloc(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                                const inkling_experts_t* experts, const uint8_t* padding_mask, void* out,
                                inkling_route_out_t* route_out, void* stream);

/*
 * Training forward: inkling_moe_forward (same out, bit for bit) that also
 * keeps, for inkling_moe_backward, the gate_up projections h = gate_up(x) in
 * fp32, the interleaved [gate, up] columns of each row, and the gate logits:
 *   saved = [T*top_k][2*I] fp32 for the routed rows, in the expert-sorted
 *           order of the routing (rows past the routed count unused), then
 *           [T][n_shared*2*I] fp32 for the shared experts, then
 *           [T][n_routed + n_shared] fp64 logits (the backward routes from
 *           them instead of recomputing them, with the same result);
 * inkling_moe_saved_size gives its size in bytes.  The caller owns `saved`
 * (device memory), and it stays valid for a backward with the same dims,
 * inputs, gate, experts and padding_mask.  The pages' layer is trained by
 * autograd, which keeps such activations between the passes.
 */
int inkling_moe_saved_size(const inkling_moe_dims_t* dims, size_t* bytes);

int inkling_moe_forward_train(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                              const inkling_experts_t* experts, const uint8_t* padding_mask, void* out,
                              void* saved, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of InklingMoE.forward: gradients of L = sum(dout * out) for the
 * layer as inkling_moe_forward computes it (chain rule through the down
 * projection, SwiGLU, the gate_up projection and the gate's log-sigmoid
 * softmax; the correction bias only moves the top-k selection and has no
 * gradient; padded tokens skip the routed experts and keep the shared ones).
 * The routing and the permutation are recomputed from x; the gate_up
 * projections are read from `saved` (written by inkling_moe_forward_train
 * with the same arguments) or, if it is NULL, recomputed, which gives the
 * same bits.  Every gradient buffer is overwritten, not accumulated; an
 * expert that receives no token gets zeros.
 *   dout [T][hidden] (dims->dtype);  dx [T][hidden] (dims->out_dtype), which
 *   must alias neither x nor dout.
 * For bf16 layers each routed slot's share of dx is rounded to fp16 before
 * the slots are summed in fp32 (like the forward's routed rows), so its
 * elements must stay below 65504 in magnitude.
 * Weight gradients have the weights' layouts.  They are accumulated in fp32
 * and stored as fp32, or, with weight_grad_dtype = INKLING_BF16, rounded once
 * to nearest-even bf16 (half the bytes written; each value is the fp32
 * gradient rounded).  A zero-initialised struct asks for fp32; any other value
 * returns INKLING_ERR_UNSUPPORTED.  d_gate_bank is always fp32.
 */
typedef struct {
    float* d_gate_bank;        /* [n_routed + n_shared][hidden] */
    void* d_routed_gate_up;    /* [n_routed][2*I][hidden]       */
    void* d_routed_down;       /* [n_routed][hidden][I]         */
    void* d_shared_gate_up;    /* [n_shared][2*I][hidden] (NULL iff n_shared == 0) */
    void* d_shared_down;       /* [n_shared][hidden][I]         */
    int32_t weight_grad_dtype; /* inkling_dtype_t of the four weight gradients */
} inkling_moe_grads_t;

int inkling_moe_backward_workspace_size(const inkling_moe_dims_t* dims, size_t* bytes);

int inkling_moe_backward(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                         const inkling_experts_t* experts, const uint8_t* padding_mask, const void* dout,
                         const void* saved, void* dx, inkling_moe_grads_t* grads, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * InklingDenseMLP (layers page): the dense SwiGLU MLP on the fused interleaved
 * gate_up layout, scaled by the module's global_scale:
 *   out = global_scale * down . (silu(gate) * up),  [gate, up] = gate_up . x
 * (reading: the page does not say where global_scale enters; it scales the
 * output, applied here to the activation, which is the same in exact
 * arithmetic).  intermediate is the dense intermediate size (InklingTextConfig
 * dense_intermediate_size, defaulting to intermediate_size = 24576).
 *   x        [T][hidden] (dtype);  gate_up [2*intermediate][hidden], row 2j =
 *   gate_j, 2j+1 = up_j;  down [hidden][intermediate];  out [T][hidden]
 *   (out_dtype; INKLING_F32 keeps the fp32 result unrounded), must not alias x.
 * Same conventions and errors as inkling_moe_forward; limits hidden % 64 == 0,
 * intermediate % 64 == 0.  With dtype INKLING_BF16 the activation is rounded
 * to fp16 and the down weights are taken as fp16, as in inkling_moe_forward.
 */
typedef struct {
    int64_t T;
    int32_t hidden;
    int32_t intermediate;
    int32_t dtype;      /* inkling_dtype_t of x and the weights */
    int32_t out_dtype;  /* inkling_dtype_t of out */
} inkling_dense_dims_t;

int inkling_dense_mlp_workspace_size(const inkling_dense_dims_t* dims, size_t* bytes);

int inkling_dense_mlp_forward(const inkling_dense_dims_t* dims, const void* x, const void* gate_up, const void* down,
                              float global_scale, void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Stage timing (instrumentation for benchmarks).  When `events` is non-NULL,
 * each later inkling_moe_forward on the calling thread records, on its stream,
 * events[0] before the first launch and events[i] after stage i:
 *   1 router logits, 2 router selection, 3 permutation (masks, scan, scatter),
 *   4 gate_up grouped GEMM + SwiGLU (routed and shared),
 *   5 routed down grouped GEMM, 6 shared down GEMM with the combine in its
 *   epilogue.  (With few tokens per expert, at most 48 on average, the shared
 *   down tiles run in stage 5 and stage 6 is the combine alone, as it is when
 *   n_shared == 0.)
 * events[] holds INKLING_STAGE_EVENTS hipEvent_t handles created by the caller
 * (a NULL entry skips that boundary); the array must stay valid until the hook
 * is cleared with NULL.  Adds no synchronisation.  Returns INKLING_ERR_INVALID_ARGUMENT if n_events is too
 * small. */
#define INKLING_STAGE_EVENTS 7
int inkling_moe_set_stage_events(void* const* events, int n_events);

/* Static text for a return code. */
const char* inkling_moe_strerror(int code);

/* The hipError_t of the last INKLING_ERR_HIP on the calling thread (0 if none). */
int inkling_moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* INKLING_MOE_H */
