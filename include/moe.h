/*
 * moe.h - C ABI of libmoe_mi355x: the forward pass of one DeepSpeed-MoE-style
 * mixture-of-experts FFN layer on one MI355X (gfx950), as hand-written HIP kernels.
 *
 * The layer ("[Review] DeepSpeed-MoE", section "What is MoE?": a Switch-Transformer
 * style layer in which a gating function sends each token to one of several expert
 * FFNs; section "Phenomenon2": Top2-MoE adds the outputs of two experts, and
 * Residual-MoE adds a fixed dense MLP to one routed expert):
 *
 *   z      = x Wg^T (+ b)                      gate logits, fp32           [T, E]
 *   p      = softmax(z) over all E experts     fp32
 *   idx    = top-k experts by z, ties to the lower expert index            [T, k]
 *   w      = p[idx]   (optionally renormalised over the k selected)        [T, k]
 *   C      = ceil(k * T * cf / E)              capacity per expert
 *   dispatch: assignments in rank-major order (all first choices, then all
 *            second choices; lower token first); an assignment keeps slot
 *            pos < C of its expert, later ones are dropped (contribute 0)
 *   FFN_e(r) = GeLU(r W1_e^T + b1_e) W2_e^T + b2_e,  GeLU exact (erf form)
 *   y[t]   = sum_j w[t,j] FFN_{idx[t,j]}(x[t]) over kept local assignments
 *            (+ MLP(x[t]) in residual mode, the PR-MoE variant)
 *
 * One GPU may hold a share of the experts: local experts [first_local_expert,
 * first_local_expert + num_local_experts). Gate, softmax and capacity are always
 * global; dispatch, FFN and combine cover local experts, so y is this share's
 * partial output and the shares of all GPUs sum to the full layer.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host). The caller allocates and
 *     owns every buffer, including the workspace; the library keeps no pointer
 *     past the call, allocates nothing and never synchronises the stream. The
 *     one exception is the expert store (moe_expert_store_*), which owns pinned
 *     host memory and device slots: its set-up calls (create, destroy,
 *     set_expert) allocate, free and synchronise the device.
 *   - Calls enqueue on `stream` and return at once (stream order). No device data
 *     is read on the host, so a sequence of calls can be captured in a hipGraph.
 *   - Argument errors are found on the host before anything is enqueued; then
 *     nothing is launched and the status says why (moe_last_error() holds detail,
 *     per thread). A failed launch returns MOE_ERR_HIP.
 *   - Outputs are fully overwritten (dropped / non-local rows included).
 *   - Results are bit-identical from run to run (no floating-point atomics).
 *   - Tensors are row-major; weights use the nn.Linear layout [out, in]. Device
 *     pointers must be 16-byte aligned; hidden and ffn must be multiples of 64.
 *   - T == 0 is a valid no-op.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, k not in {1,2}, k > E, cf <= 0, ... */
  MOE_ERR_UNSUPPORTED = 2,        /* valid layer the kernels do not cover (H % 64 != 0, ...) */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP launch or runtime call failed */
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_F16 = 1, MOE_DTYPE_BF16 = 2 } moe_dtype_t;

/* "DeepSpeed-MoE Inference" wiki page, section on PR-MoE: the model type is
 * 'standard' or 'residual'; residual adds a dense MLP to one routed expert. */
typedef enum { MOE_MLP_STANDARD = 0, MOE_MLP_RESIDUAL = 1 } moe_mlp_type_t;

/* Divide the k combine weights of a token by their sum (before drops). Off by
 * default: the combine weight is the raw softmax probability of the expert. */
#define MOE_FLAG_RENORM_TOPK 1u
/* Decode-sized batches (the path where the first expert kernel routes the batch
 * itself): run both expert products in one launch, the hidden rows handed from
 * the W1 work-groups to the W2 work-groups through memory inside the launch
 * ("DeepSpeed Inference" review, proposed-method section: fusing the operators
 * of small batches into few kernels). Same results bit for bit; ignored where
 * moe_layer_plan does not report experts_one_launch. Off by default: on MI355X
 * the two-launch form measures as fast or faster. */
#define MOE_FLAG_DECODE_ONE_LAUNCH 2u

typedef struct {
  int64_t num_tokens;          /* T >= 0 */
  int32_t hidden;              /* H, multiple of 64 */
  int32_t ffn;                 /* F (expert and dense-MLP width), multiple of 64 */
  int32_t num_experts;         /* E >= 1: gate width and capacity denominator, <= 512 */
  int32_t first_local_expert;  /* e_lo, 0 <= e_lo < E */
  int32_t num_local_experts;   /* E_loc >= 1, e_lo + E_loc <= E */
  int32_t top_k;               /* 1 or 2, <= E */
  double capacity_factor;      /* finite and > 0 */
  moe_mlp_type_t mlp_type;     /* RESIDUAL requires top_k == 1 */
  moe_dtype_t dtype;           /* activations, weights and output; accumulation is fp32 */
  uint32_t flags;              /* MOE_FLAG_* */
} moe_layer_desc_t;

typedef struct {
  const void* gate_w;          /* [E, H] dtype */
  const float* gate_b;         /* [E] fp32, or NULL for no gate bias */
  const void* w1;              /* [E_loc, F, H] dtype */
  const void* b1;              /* [E_loc, F]    dtype */
  const void* w2;              /* [E_loc, H, F] dtype */
  const void* b2;              /* [E_loc, H]    dtype */
  const void* mlp_w1;          /* residual only: [F, H]; else ignored (may be NULL) */
  const void* mlp_b1;          /* residual only: [F] */
  const void* mlp_w2;          /* residual only: [H, F] */
  const void* mlp_b2;          /* residual only: [H] */
  /* Optional per-expert placement, all four set or all NULL. Each is a DEVICE
   * array of E_loc pointers: local expert i's W1 [F, H] starts at w1_experts[i],
   * its b1 [F] at b1_experts[i], W2 [H, F] at w2_experts[i], b2 [H] at
   * b2_experts[i]. A pointer may address device memory or pinned host memory
   * (hipHostMalloc) that the device reads directly over the host link; the expert
   * kernels read only the experts the routing selects. When set, w1 / b1 / w2 /
   * b2 above are ignored and may be NULL. Every pointer must be 16-byte aligned
   * and stay valid until the work enqueued with it has run (moe_expert_store_t
   * below maintains such tables). */
  const void* const* w1_experts;
  const void* const* b1_experts;
  const void* const* w2_experts;
  const void* const* b2_experts;
} moe_layer_weights_t;

/* Capacity C = ceil(k * T * cf / E) (host, pure), computed exactly from the
 * binary value of cf (saturates at INT64_MAX). The pages print no formula;
 * this is the plainest reading, with the global expert count and no floor.
 * Returns -1 for invalid arguments: T < 0, E outside [1, 512], k outside
 * {1, 2}, T * k > 2^30, cf not finite or <= 0 (the descriptor's limits). */
int64_t moe_capacity(int64_t T, int32_t E, int32_t k, double cf);

/* R_max = min(E_loc * C, k * T): rows of the dispatched buffers (host, pure).
 * Returns -1 if the descriptor is invalid. */
int64_t moe_max_rows(const moe_layer_desc_t* d);

/* Workspace bytes that moe_layer_forward needs for this descriptor (host). Also
 * enough for every step entry point below. */
moe_status_t moe_workspace_size(const moe_layer_desc_t* d, size_t* bytes /* host */);

/* How moe_layer_forward runs a descriptor (host, pure). */
typedef enum { MOE_GATE_VECTOR = 0, MOE_GATE_MATRIX = 1 } moe_gate_path_t;
typedef enum {
  MOE_EXPERTS_GROUPED_GEMM = 0,  /* matrix-core grouped GEMMs over the expert segments */
  MOE_EXPERTS_STREAM = 1         /* segments of <= 8 rows: two weight-streaming kernels */
} moe_expert_path_t;
typedef struct {
  int64_t capacity;              /* C */
  int64_t max_rows;              /* R_max */
  size_t workspace_bytes;
  moe_gate_path_t gate_path;
  moe_expert_path_t expert_path;
  int32_t dispatch_in_expert_kernel;  /* 1: the first expert kernel routes the batch itself */
  int32_t combine_in_expert_kernel;   /* 1: the last expert kernel writes y (top-1, standard) */
  int32_t dense_in_expert_kernels;    /* 1: the residual MLP's tiles run inside the expert GEMMs */
  int32_t launches;                   /* kernel launches of one moe_layer_forward */
  int32_t tile_rows;                  /* grouped GEMM: rows per tile (0 on the streaming path) */
  int32_t tile_cols_w1, tile_cols_w2; /* grouped GEMM: columns per tile of the two products */
  int32_t experts_one_launch;         /* 1: both expert products (and the routing) in one launch */
} moe_layer_plan_t;
moe_status_t moe_layer_plan(const moe_layer_desc_t* d, moe_layer_plan_t* out /* host */);

/* Gate (steps z, p, idx, w above): x [T, H] dtype -> topk_idx [T, k] int32,
 * topk_w [T, k] fp32, and, when probs != NULL, probs [T, E] fp32. Logits,
 * softmax and the top-k choice are computed in fp32; ties go to the lower index.
 * Softmax-based routing: "Fast MoE Inference via Predictive Prefetching and
 * Expert Replication", problem statement. */
moe_status_t moe_gate(const moe_layer_desc_t* d, const void* x, const void* gate_w,
                      const float* gate_b, int32_t* topk_idx, float* topk_w, float* probs,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* Dispatch (capacity and rank-major drops), atomic-free: per-block counts,
 * column scan, stable in-block ranks. "[Review] DeepSpeed-MoE", section "What is
 * MoE?": the gating function sends each token to the expert it selects, so the
 * tokens of one expert are gathered into that expert's segment before its FFN
 * runs. The pages give no capacity rule or drop order: the capacity
 * C = ceil(k T cf / E) and the rank-major priority (all first choices before
 * any second choice, lower token first) are the plainest readings, and a
 * dropped assignment contributes nothing. From topk_idx [T, k] int32 (values in
 * [0, E); others count as no expert) writes:
 *   expert_demand  [E]        assignments per global expert (all, kept or not)
 *   expert_offsets [E_loc+1]  exclusive scan of kept rows per local expert
 *   slot_token     [R_max]    token of each dispatched row, -1 past the last row
 *   token_slot     [T, k]     row of each assignment, -1 if dropped or non-local
 *   x_disp         [R_max, H] dtype, gathered x rows (zero past the last row)
 * x_disp may be NULL to skip the gather. */
moe_status_t moe_dispatch(const moe_layer_desc_t* d, const int32_t* topk_idx, const void* x,
                          int32_t* expert_demand, int32_t* expert_offsets, int32_t* slot_token,
                          int32_t* token_slot, void* x_disp, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Expert FFN over the dispatched rows, grouped by local expert:
 * y_disp[r] = GeLU(x_disp[r] W1_e^T + b1_e) W2_e^T + b2_e for r in segment e
 * ([expert_offsets[e], expert_offsets[e+1])). The hidden activation is rounded to
 * dtype; accumulation is fp32; y_disp [R_max, H] is fp32 (rows past the last
 * dispatched row are left unspecified). "[Review] DeepSpeed-MoE", "What is MoE?":
 * the experts are FFNs; the page's model table fixes F = 4H for its models. */
moe_status_t moe_expert_ffn(const moe_layer_desc_t* d, const void* x_disp,
                            const int32_t* expert_offsets, const moe_layer_weights_t* w,
                            float* y_disp, void* ws, size_t ws_bytes, hipStream_t stream);

/* Dense MLP of the residual (PR-MoE) variant over all T tokens:
 * out [T, H] fp32 = GeLU(x W1^T + b1) W2^T + b2 with the mlp_* weights.
 * ("[Review] DeepSpeed-MoE", "Phenomenon2": Residual-MoE keeps a fixed MLP.) */
moe_status_t moe_dense_ffn(const moe_layer_desc_t* d, const void* x, const moe_layer_weights_t* w,
                           float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Combine: y[t] = sum over j with token_slot[t,j] >= 0 of topk_w[t,j] * y_disp[token_slot[t,j]]
 * (+ dense_out[t] when dense_out != NULL), summed in fp32 in choice order and
 * rounded once to dtype. y [T, H] is fully written; a token with nothing kept
 * gets 0 (or dense_out[t]). "[Review] DeepSpeed-MoE", section "PR-MoE: Pyramid-
 * Residual-MoE", part "Phenomenon2": Top2-MoE adds the outputs of the two
 * experts a token is sent to, and Residual-MoE adds the output of a fixed MLP to
 * that of the one routed expert; the gate-probability weight w on each expert
 * term follows the gated mixture of "What is MoE?" (a Switch-Transformer layer).
 * Arguments: y_disp [R_max, H] fp32 (rows of moe_expert_ffn), token_slot [T, k]
 * int32 from moe_dispatch (values >= R_max are an error of the caller, never
 * checked on the device), topk_w [T, k] fp32, dense_out [T, H] fp32 or NULL,
 * y [T, H] dtype. Errors: INVALID_ARGUMENT for NULL or misaligned pointers. */
moe_status_t moe_combine(const moe_layer_desc_t* d, const float* y_disp, const int32_t* token_slot,
                         const float* topk_w, const float* dense_out, void* y, hipStream_t stream);

/* The whole layer: x [T, H] dtype -> y [T, H] dtype, using ws of at least
 * moe_workspace_size() bytes. In residual mode the dense MLP runs too. The
 * layer is the MoE FFN of "[Review] DeepSpeed-MoE", section "What is MoE?" (a
 * gate picks experts per token, each expert is an FFN, the outputs are mixed by
 * the gate), in the Top2-MoE and Residual-MoE forms of "Phenomenon2" (section
 * "PR-MoE: Pyramid-Residual-MoE"); the 'standard' / 'residual' choice is the
 * mlp_type option of the "DeepSpeed-MoE Inference" wiki page (section on PR-MoE),
 * and a share of the experts is the expert-parallel placement of that page's
 * inference set-up. Ownership: x, y, the weights and ws belong to the caller;
 * ws holds the intermediates (logits, routing, h, y_disp) and may be reused
 * after the work enqueued on stream has run. Errors: INVALID_ARGUMENT (NULL or
 * misaligned pointers, bad descriptor), UNSUPPORTED, WORKSPACE_TOO_SMALL, all
 * found before anything is enqueued; MOE_ERR_HIP when a launch fails. */
moe_status_t moe_layer_forward(const moe_layer_desc_t* d, const moe_layer_weights_t* w,
                               const void* x, void* y, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* Bytes of the device scratch array that moe_layer_forward_noalloc uses in
 * place of a workspace (one copy per GPU, held until the process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES (128u << 20)

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, serving loops, harnesses
 * that forbid allocation): the intermediates live in the library's own device
 * scratch array of MOE_NOALLOC_SCRATCH_BYTES per GPU (enough for every layer
 * whose moe_workspace_size is at most that, e.g. 8- to 4096-token batches of
 * the 350M / 1.3B +MoE-128 shapes), so the call allocates nothing. The caller
 * still owns x, y and the weights. Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (on different streams, or from several
 * threads without ordering) race and give wrong results; calls ordered on one
 * stream are fine. Errors: as moe_layer_forward, and WORKSPACE_TOO_SMALL when
 * the layer needs more than MOE_NOALLOC_SCRATCH_BYTES (found before anything
 * is enqueued). */
moe_status_t moe_layer_forward_noalloc(const moe_layer_desc_t* d, const moe_layer_weights_t* w,
                                       const void* x, void* y, hipStream_t stream);

/* Optional timing hook for moe_layer_forward_ex. Any non-NULL event of the first
 * group is recorded on the stream right before / after the phase (gate, dispatch,
 * expert FFN, combine); ffn_split is recorded between the two expert kernels (after
 * the W1 kernel, before the W2 kernel). The residual mode's dense MLP runs inside
 * the two expert GEMMs when moe_layer_plan reports dense_in_expert_kernels, else
 * after the W2 kernel (inside the ffn_split .. ffn_end window).
 * The second group is recorded by the launch of the expert kernels themselves
 * (the dispatch's own start and end timestamps): up_* for the W1 kernel, down_*
 * for the W2 kernel. Events must come from hipEventCreate (timing enabled). */
typedef struct {
  hipEvent_t gate_begin, gate_end;
  hipEvent_t dispatch_begin, dispatch_end;
  hipEvent_t ffn_begin, ffn_split, ffn_end;
  hipEvent_t combine_begin, combine_end;
  hipEvent_t up_start, up_stop, down_start, down_stop;
} moe_phase_events_t;

/* moe_layer_forward with phase events (ev may be NULL: then identical to it). */
moe_status_t moe_layer_forward_ex(const moe_layer_desc_t* d, const moe_layer_weights_t* w,
                                  const void* x, void* y, void* ws, size_t ws_bytes,
                                  hipStream_t stream, const moe_phase_events_t* ev);

/* ---- Host-resident experts with a device cache (for callers whose experts do
 * not all fit in HBM). "[Review] DeepSpeed-MoE", PR-MoE / MoS section: the
 * weights of the many experts are the memory cost of MoE inference; "Fast MoE
 * Inference via Predictive Prefetching and Expert Replication": keep experts off
 * the GPU and bring in the ones the routing selects.
 *
 * A store owns pinned host memory holding all E_loc local experts of one layer
 * and `slots` device slots caching some of them, plus the per-expert pointer
 * tables that moe_expert_store_weights() puts into a moe_layer_weights_t. The
 * expert kernels read a cached expert from its slot and any other expert
 * directly from pinned host memory over the host link, only when the routing
 * selects it. create / destroy / set_expert synchronise the device (set-up
 * calls); update, update_async and commit only enqueue work. Use one store from
 * one compute stream at a time. */
typedef struct moe_expert_store* moe_expert_store_t;

/* Allocates the store for descriptor d (pinned host memory for E_loc experts,
 * `slots` in [0, E_loc] device slots). All experts start host-resident with
 * zero weights; *out receives the handle (NULL on error). */
moe_status_t moe_expert_store_create(const moe_layer_desc_t* d, int32_t slots, moe_expert_store_t* out /* host */);

/* Frees everything the store owns (after a device synchronisation). NULL is a no-op. */
moe_status_t moe_expert_store_destroy(moe_expert_store_t store);

/* Copies local expert e's weights (HOST pointers, nn.Linear layout: W1 [F, H],
 * b1 [F], W2 [H, F], b2 [H], dtype of the descriptor) into the store, and into
 * its slot when it is cached. */
moe_status_t moe_expert_store_set_expert(moe_expert_store_t store, int32_t e, const void* w1, const void* b1,
                                         const void* w2, const void* b2);

/* Points w's per-expert tables at the store (w1 / b1 / w2 / b2 are set to NULL;
 * the caller fills the gate and, in residual mode, the dense MLP weights). */
moe_status_t moe_expert_store_weights(moe_expert_store_t store, moe_layer_weights_t* w /* host */);

/* Folds demand (HOST array [E] of assignments per global expert, e.g. a host
 * copy of moe_dispatch's expert_demand) into each local expert's score
 * (score = 0.5 * score + demand) and keeps the `slots` best-scoring experts
 * (score > 0, ties to the lower index) in the device slots. Enqueued on stream:
 * leaving experts switch to host reads, incoming experts are copied into their
 * slots, then switch to slot reads; work enqueued earlier on the stream uses the
 * old placement. *copied (may be NULL) receives the number of experts copied. */
moe_status_t moe_expert_store_update(moe_expert_store_t store, const int32_t* demand /* host */,
                                     hipStream_t stream, int32_t* copied /* host */);

/* The same choice as moe_expert_store_update, with the copies on copy_stream so
 * that they overlap with work enqueued on stream meanwhile (MoE-MPMC summary:
 * expert loads overlapped with inference). Enqueued: on stream, leaving experts
 * switch to host reads; copy_stream waits for that point of stream and copies
 * the incoming experts into their slots. Until moe_expert_store_commit, every
 * incoming expert is still read from host memory, so results never depend on
 * when the copies finish. A pending asynchronous update is committed (on
 * stream) by the next update, update_async or commit. copy_stream must differ
 * from stream; the library creates no stream (give both the default priority).
 * Errors: INVALID_ARGUMENT (NULL store or demand, equal streams, negative
 * demand), MOE_ERR_HIP. */
moe_status_t moe_expert_store_update_async(moe_expert_store_t store, const int32_t* demand /* host */,
                                           hipStream_t stream, hipStream_t copy_stream,
                                           int32_t* copied /* host */);

/* Ends a pending update_async: stream waits for its copies, then the copied
 * experts switch to slot reads for the work enqueued after. Nothing pending: a
 * no-op. */
moe_status_t moe_expert_store_commit(moe_expert_store_t store, hipStream_t stream);

/* slot_of[i] (HOST array [E_loc]) = device slot of local expert i, or -1 if it
 * is read from host memory, as chosen by the last update call (after an
 * update_async, reads switch to the slot at the commit). */
moe_status_t moe_expert_store_residency(moe_expert_store_t store, int32_t* slot_of /* host */);

/* Static text for a status code. */
const char* moe_status_str(moe_status_t st);

/* Detail of the last error on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
