/*
 * swimba.h - C ABI of the Swimba (Switch Mamba) mixer forward pass on MI355X.
 *
 * The method: arXiv 2603.06938, "Swimba: Switch Mamba Model Scales State
 * Space Models". Per token a router gives softmax weights over E experts and
 * keeps the top-k; each selected expert's linear projection emits its own
 * B, C and X streams; these are mixed in parameter space into one injection
 * U~_t = sum_j pi_{t,j} B_{t,j} X_{t,j}^T and one readout C~_t; one state per
 * head then runs h_t = a_h h_{t-1} + U~_t, y_t = C~_t^T h_t with a scalar,
 * contractive a_h shared by all experts and all steps.
 * (papernotes.org notes on the paper, Method, key designs 1 and 2; gist.science
 *  English summary, Technical Summary section 2, Architecture Details.)
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers unless a comment says otherwise. Tensors are
 *    dense, row-major, with the shapes given below. Every device pointer must be
 *    16-byte aligned.
 *  - Token index m = b * seqlen + t.
 *  - The caller owns every buffer, including the workspace, whose size comes
 *    from swimba_workspace_size(). The library never allocates or frees device
 *    memory and keeps no device state between calls.
 *  - Work is enqueued on the given stream only (never the null stream, unless
 *    the caller passes it); no call synchronises.
 *  - Errors: a call validates every argument before it launches anything. On
 *    an error it returns a negative swimba_status, launches nothing, leaves
 *    every output untouched and records a message for swimba_last_error().
 *    A failed kernel launch returns SWIMBA_ERR_HIP. No C++ exception crosses
 *    this boundary.
 *  - Same inputs give bitwise-identical outputs (no order-dependent atomics).
 *  - Calls that share a workspace, or write the same outputs, must not run
 *    concurrently.
 */
#ifndef SWIMBA_H
#define SWIMBA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWIMBA_ABI_VERSION 1

/*
 * Element types. "stream" below names the element type of the intermediate
 * streams B_hat, X_hat and C_mix:
 *   SWIMBA_F32:  u, weights, streams and y are float32.
 *   SWIMBA_BF16: u, weights and y are bfloat16; the streams are float16 (the
 *                same bytes with 8x finer spacing, so three roundings of the
 *                streams do not dominate the error of y; their magnitudes, and
 *                those of C_mix . B_hat dot products, must stay below 65504).
 * States and a are float32 in both cases.
 */
typedef enum swimba_dtype {
  SWIMBA_F32 = 0,
  SWIMBA_BF16 = 1
} swimba_dtype;

typedef enum swimba_status {
  SWIMBA_OK = 0,
  SWIMBA_ERR_NULL = -1,        /* a required pointer is NULL */
  SWIMBA_ERR_DIMS = -2,        /* a dimension is out of range or inconsistent */
  SWIMBA_ERR_UNSUPPORTED = -3, /* valid, but no kernel exists for this shape */
  SWIMBA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  SWIMBA_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned */
  SWIMBA_ERR_HIP = -6          /* a HIP runtime call or kernel launch failed */
} swimba_status;

typedef enum swimba_call {
  SWIMBA_CALL_ROUTE = 0,
  SWIMBA_CALL_PROJECT = 1,
  SWIMBA_CALL_SCAN = 2,
  SWIMBA_CALL_DECODE = 3,
  SWIMBA_CALL_SCAN_BACKWARD = 4,
  SWIMBA_CALL_PROJECT_BACKWARD = 5,
  SWIMBA_CALL_PROJECT_BACKWARD_SAVED = 6,
  SWIMBA_CALL_SEPARATED = 7
} swimba_call;

/*
 * Dimensions. Constraints checked by every call:
 *   batch >= 0, seqlen >= 0 (M = batch*seqlen may be 0), d_model >= 1,
 *   nheads >= 1, headdim >= 1, dstate >= 1, ngroups >= 1 and divides nheads,
 *   n_experts >= 1, 1 <= top_k <= n_experts, chunk >= 1, dtype in swimba_dtype.
 * Shapes with a kernel (else SWIMBA_ERR_UNSUPPORTED):
 *   headdim == 64; dstate in {16, 32, 64, 128}; d_model % 32 == 0;
 *   n_experts <= 256; top_k <= 8 (the prefill scans: top_k <= 4 for bf16,
 *   <= 2 for fp32; the scan backward: top_k <= 2);
 *   chunk in {32, 64, 128, 256} for the scan.
 * Sizes the kernels can address (else SWIMBA_ERR_DIMS, before any launch;
 * 2 GiB here means 0x7FFFFFF0 bytes, so that the byte offset 2^31 the kernels
 * give to loads that must read zeros lies past every buffer): u at most 2 GiB
 * in every call that reads it; w_router and each expert's [W, D] weight
 * matrix at most 2 GiB; in the scans, one sequence's B_hat and X_hat
 * (T * k * G*N and T * k * H*P stream elements) and its intra-chunk Gram
 * tiles at most 2 GiB (a longer sequence is scanned in pieces, the state
 * handed on through h_final and h_init).
 */
typedef struct swimba_dims {
  int32_t batch;      /* Bt: independent sequences */
  int32_t seqlen;     /* T: tokens per sequence (1 for a decode step) */
  int32_t d_model;    /* D: width of the mixer input u_t */
  int32_t nheads;     /* H */
  int32_t headdim;    /* P: X and y width per head */
  int32_t dstate;     /* N: state rows per head (state is N x P) */
  int32_t ngroups;    /* G: B and C groups; head h uses group h / (H/G) */
  int32_t n_experts;  /* E */
  int32_t top_k;      /* k: selected experts per token */
  int32_t chunk;      /* L: SSD chunk length (scan only) */
  int32_t dtype;      /* swimba_dtype */
  int32_t reserved;   /* must be 0 */
} swimba_dims;

int32_t swimba_abi_version(void);

/* Message of the last failed call on this host thread (host memory, owned by
 * the library, valid until the next call on this thread). */
const char* swimba_last_error(void);

/* Workspace bytes that call `call` needs for `dims` (0 if none). Returns 0
 * for invalid dims as well; the call itself then reports the error. */
size_t swimba_workspace_size(const swimba_dims* dims, int32_t call);

/*
 * Router and top-k active set.
 * (papernotes.org notes, Method, key design 1: pi_t = softmax(g_t), K_t a
 *  top-k set; gist.science English summary, section 2, Expert Routing.)
 * g_t = W_r u_t accumulated in fp32 (never rounded to bf16); pi_t = softmax
 * over all E logits in fp32; K_t = the k largest logits, descending, exact
 * ties to the lower expert index; topk_w[m, j] = pi_{m, K_t[j]} (not
 * renormalised).
 *   u         [M, D]   dtype
 *   w_router  [E, D]   dtype
 *   topk_idx  [M, k]   int32 out
 *   topk_w    [M, k]   float32 out
 *   logits    [M, E]   float32 out, or NULL
 */
swimba_status swimba_route_topk(const swimba_dims* dims, const void* u, const void* w_router,
                                int32_t* topk_idx, float* topk_w, float* logits,
                                hipStream_t stream);

/*
 * Expert projections with the parameter-space mix in the epilogue.
 * (papernotes.org notes, Method, key design 1: each expert's linear
 *  projection of the token gives B^(e), C^(e), X^(e); mixing equation for
 *  U~_t and C~_t. gist.science English summary, section 2, Parameter Mixing.)
 * For slot j of token m with expert e = topk_idx[m, j] and weight w:
 *   z = W_e u_m (fp32 accumulation), W_e = w_experts[e], rows X | B | C;
 *   X_hat[m, j] = z[0 : H*P]                          (as [H, P])
 *   B_hat[m, j] = w * z[H*P : H*P + G*N]              (as [G, N])
 *   C_mix[m]    = sum_j w * z[H*P + G*N : H*P + 2*G*N] (as [G, N]), summed in
 *                 slot order j = 0..k-1 in fp32, then stored as stream.
 * U~_m = sum_j B_hat[m, j] X_hat[m, j]^T is never formed.
 *   u          [M, D]              dtype
 *   w_experts  [E, H*P + 2*G*N, D] dtype
 *   topk_idx   [M, k] int32 (values in [0, E); validated on the device: an
 *              out-of-range index makes its slot contribute zeros)
 *   topk_w     [M, k] float32
 *   B_hat      [M, k, G, N] stream out
 *   X_hat      [M, k, H, P] stream out
 *   C_mix      [M, G, N]    stream out
 *   ws         workspace of swimba_workspace_size(dims, SWIMBA_CALL_PROJECT)
 */
swimba_status swimba_expert_project_mix(const swimba_dims* dims, const void* u,
                                        const void* w_experts, const int32_t* topk_idx,
                                        const float* topk_w, void* B_hat, void* X_hat,
                                        void* C_mix, void* ws, size_t ws_bytes,
                                        hipStream_t stream);

/*
 * Single-trajectory scan, solved in chunks of L tokens (SSD).
 * (papernotes.org notes, Method, key design 1 state equation and the reuse of
 *  the chunked SSD solver; key design 2: A shared over experts and steps.)
 * For every sequence b and head h (group g = h / (H/G)), with h_{-1} = h_init:
 *   h_t = a_h h_{t-1} + sum_j B_hat[t, j, g] X_hat[t, j, h]^T      (N x P)
 *   y[t, h] = C_mix[t, g]^T h_t                                     (P)
 * computed as, per chunk: a masked quadratic form over the chunk's
 * k-concatenated (token, slot) pairs, plus the decayed readout of the state
 * entering the chunk; states are carried across chunks in fp32. Matrix-core
 * operands are of the stream type, accumulation is fp32.
 *   B_hat    [M, k, G, N] stream;  X_hat [M, k, H, P] stream;  C_mix [M, G, N] stream
 *   a        [H] float32, each in [0, 1)
 *   h_init   [Bt, H, N, P] float32, or NULL for zeros
 *   y        [M, H, P] dtype out
 *   h_final  [Bt, H, N, P] float32 out, or NULL (may alias h_init)
 *   ws       workspace of swimba_workspace_size(dims, SWIMBA_CALL_SCAN)
 */
swimba_status swimba_ssd_chunk_scan(const swimba_dims* dims, const void* B_hat,
                                    const void* X_hat, const void* C_mix, const float* a,
                                    const float* h_init, void* y, float* h_final, void* ws,
                                    size_t ws_bytes, hipStream_t stream);

/*
 * One recurrent decode step for `batch` sequences (dims->seqlen must be 1).
 * (papernotes.org notes, Method, key design 1, the recurrent form; key
 *  findings: token-by-token decoding.)
 * Routes u, projects the k selected experts, updates the state in place,
 *   h <- a_h h + sum_j B_hat_j X_hat_j^T  (fp32),   y = C_mix^T h,
 * and reads out y.
 *   u         [Bt, D] dtype;  w_router [E, D] dtype;  w_experts as above
 *   a         [H] float32
 *   h         [Bt, H, N, P] float32, in/out
 *   y         [Bt, H, P] dtype out
 *   topk_idx  [Bt, k] int32 out, or NULL
 *   ws        workspace of swimba_workspace_size(dims, SWIMBA_CALL_DECODE)
 */
swimba_status swimba_decode_step(const swimba_dims* dims, const void* u, const void* w_router,
                                 const void* w_experts, const float* a, float* h, void* y,
                                 int32_t* topk_idx, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * swimba_decode_step for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same kernels and the same results, with the
 * workspace in a static scratch array of 32 MiB per device that the library
 * holds until the process ends (its address is looked up on the first call
 * on each device; the calling thread's current device must own `stream`).
 * Dims whose decode workspace (swimba_workspace_size(dims,
 * SWIMBA_CALL_DECODE)) exceeds 32 MiB return SWIMBA_ERR_WORKSPACE before any
 * launch. Every call on one device shares that scratch: calls that overlap
 * on one device (other streams, other threads) race and must be serialised
 * by the caller. Allocates nothing (no hipMalloc, no hipFree). Arguments and
 * errors otherwise as for swimba_decode_step.
 */
swimba_status swimba_decode_step_noalloc(const swimba_dims* dims, const void* u,
                                         const void* w_router, const void* w_experts,
                                         const float* a, float* h, void* y, int32_t* topk_idx,
                                         hipStream_t stream);

/*
 * Output projection of the mixer: the single projection that follows the
 * recurrence (gist.science English summary, Technical Summary section 2,
 * Architecture Details, the state-update equation "followed by a single
 * output projection"), read as Mamba-2's projection from the H*P readout
 * back to d_model: out[m, :] = W_out y[m, :], fp32 accumulation, out rounded
 * to dtype. No bias.
 *   y      [M, H*P] dtype   (the y of swimba_ssd_chunk_scan / swimba_decode_step)
 *   w_out  [D, H*P] dtype   (D = d_model)
 *   out    [M, D]   dtype out (must not overlap y or w_out)
 * Uses dims.batch, seqlen, d_model, nheads, headdim and dtype (M = batch *
 * seqlen). No workspace. Errors as for the other calls.
 */
swimba_status swimba_output_project(const swimba_dims* dims, const void* y, const void* w_out,
                                    void* out, hipStream_t stream);

/*
 * Expert-mixed diagonal transition (papernotes.org notes, Limitations and
 * outlook: the parameter-space mix extended to the transition's diagonal,
 * keeping the contraction). Each expert e has a per-head decay a_experts[e, h]
 * in [0, 1]; a token's decay is their convex mix over its selected experts,
 * the routing weights renormalised over the k slots (slot order, fp32):
 *   a[t, h] = sum_j w[t, j] a_experts[idx[t, j], h] / sum_j w[t, j]
 * (an index outside [0, E) adds decay 0 with its weight). Equal expert decays
 * give back the shared decay. The three calls below use it.
 *
 * swimba_mix_decay writes what the mixed scan consumes: per sequence b, head h
 * and token t of a chunk starting at c0 (chunks of dims.chunk tokens),
 *   log_decay[b, h, t] = sum_{u = c0}^{t} max(log2 a[u, h], -126)
 * (a running log2 decay within the chunk; a zero decay counts as 2^-126).
 *   topk_idx   [M, k] int32;  topk_w [M, k] float32 (from swimba_route_topk)
 *   a_experts  [E, H] float32
 *   log_decay  [Bt, H, T] float32 out
 * No workspace. chunk must be 32, 64, 128 or 256.
 */
swimba_status swimba_mix_decay(const swimba_dims* dims, const int32_t* topk_idx,
                               const float* topk_w, const float* a_experts, float* log_decay,
                               hipStream_t stream);

/*
 * swimba_ssd_chunk_scan with the expert-mixed decay: the same recurrence with
 * the decay of token t, h_t = a[t, h] h_{t-1} + sum_j B_hat X_hat^T, given as
 * the log_decay of swimba_mix_decay for the same dims (same chunk). Every
 * other argument, the workspace and the errors are those of
 * swimba_ssd_chunk_scan.
 *   log_decay  [Bt, H, T] float32 (may be NULL only when seqlen is 0)
 */
swimba_status swimba_ssd_chunk_scan_mixed(const swimba_dims* dims, const void* B_hat,
                                          const void* X_hat, const void* C_mix,
                                          const float* log_decay, const float* h_init, void* y,
                                          float* h_final, void* ws, size_t ws_bytes,
                                          hipStream_t stream);

/*
 * swimba_decode_step with the expert-mixed decay: each sequence's decay is
 * mixed from a_experts [E, H] float32 with this step's routing. Every other
 * argument, the workspace (SWIMBA_CALL_DECODE) and the errors are those of
 * swimba_decode_step.
 */
swimba_status swimba_decode_step_mixed(const swimba_dims* dims, const void* u,
                                       const void* w_router, const void* w_experts,
                                       const float* a_experts, float* h, void* y,
                                       int32_t* topk_idx, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/*
 * Backward of swimba_ssd_chunk_scan (papernotes.org notes, Experiments: the
 * converted model is fine-tuned, which needs the gradients through the
 * recurrence). For the loss l(y, h_final) with dy = dl/dy and dh_final =
 * dl/dh_final, and g_t = dl/dh_t (g_t = C_mix_t dy_t^T + a g_{t+1}, g_T =
 * dh_final):
 *   dX_hat[t, j, h]  = g_t[h]^T B_hat[t, j, g]                      (P)
 *   dB_hat[t, j, g]  = sum_{h in group g} g_t[h] X_hat[t, j, h]        (N)
 *   dC_mix[t, g]     = sum_{h in group g} h_t[h] dy[t, h]             (N)
 *   da[h]            = sum_t <g_t[h], h_{t-1}[h]>,   dh_init = a g_0
 * solved in chunks of 64 tokens (32 for float32 problems) whatever
 * dims->chunk is: local chunk states on matrix cores, a sweep over chunks for
 * the states entering each chunk from either side, and the within-chunk
 * quadratic forms on matrix cores (for bf16 problems fp16 operands, dy and
 * the states under power-of-two scales; float32 operands for float32
 * problems; fp32 accumulation). For bf16 problems the chunk states cross HBM
 * in the workspace as fp16 (rows of P elements for the entering states),
 * each under a power-of-two factor; the sweep sums in fp32. Sums over heads
 * and chunks run in a fixed order, so results are deterministic.
 *   B_hat, X_hat, C_mix, a, h_init   as given to swimba_ssd_chunk_scan
 *   dy        [M, H, P] dtype
 *   dh_final  [Bt, H, N, P] float32, or NULL for zeros
 *   dB_hat    [M, k, G, N] float32 out;  dX_hat [M, k, H, P] float32 out
 *   dC_mix    [M, G, N] float32 out;  da [H] float32 out
 *   dh_init   [Bt, H, N, P] float32 out, or NULL
 *   ws        workspace of swimba_workspace_size(dims, SWIMBA_CALL_SCAN_BACKWARD)
 * Shapes and errors as for swimba_ssd_chunk_scan, with top_k <= 2.
 */
swimba_status swimba_ssd_chunk_scan_backward(const swimba_dims* dims, const void* B_hat,
                                             const void* X_hat, const void* C_mix,
                                             const float* a, const float* h_init, const void* dy,
                                             const float* dh_final, float* dB_hat, float* dX_hat,
                                             float* dC_mix, float* da, float* dh_init, void* ws,
                                             size_t ws_bytes, hipStream_t stream);

/*
 * Backward of the router, the expert projections and the parameter-space mix
 * (papernotes.org notes on "Swimba: Switch Mamba Model Scales State Space
 * Models", Method, key design 1: z_j = W^(e_j) u with rows X | B | C,
 * B_hat_j = w_j B_j, C_mix = sum_j w_j C_j, w_j = softmax(W_r u)[e_j];
 * Experiments: fine-tuning needs these gradients). Given the gradients of
 * the scan's inputs (from swimba_ssd_chunk_scan_backward):
 *   dz_j      = [dX_hat_j | w_j dB_hat_j | w_j dC_mix]
 *   dw_j      = <B_j, dB_hat_j> + <C_j, dC_mix>
 *   dg        = pi * (dpi - <pi, dpi>),  dpi = dw scattered to the selected experts
 *   du        = sum_j W^(e_j)^T dz_j + W_r^T dg
 *   dW_experts[e] = sum over the (token, slot) pairs routed to e of dz_j u^T
 *   dW_router = dg^T u
 * The top-k set has no gradient (it is piecewise constant in the logits).
 * The call recomputes the forward routing and projection with the forward's
 * own kernels (same bits as swimba_route_topk + swimba_expert_project_mix),
 * so only the primal inputs are passed. du and dW_experts are grouped GEMMs
 * on matrix cores over the pairs sorted by expert (bf16 operands, or float32;
 * fp32 accumulation); every sum over slots, pairs and tokens runs in a fixed
 * order, so results are deterministic.
 *   u, w_router, w_experts   as given to the forward calls (dtype)
 *   dB_hat      [M, k, G, N] float32;  dX_hat [M, k, H, P] float32
 *   dC_mix      [M, G, N] float32
 *   du          [M, D] float32 out
 *   dW_router   [E, D] float32 out;  dW_experts [E, W, D] float32 out
 *               (zeros when M is 0; every other pointer may then be NULL)
 *   ws          workspace of swimba_workspace_size(dims, SWIMBA_CALL_PROJECT_BACKWARD)
 * Shapes and errors as for swimba_expert_project_mix; in addition
 * M * k * (H*P + 2*G*N) and M * k * D elements of the input type must stay
 * below 2^31 bytes (SWIMBA_ERR_DIMS).
 */
swimba_status swimba_expert_project_mix_backward(
    const swimba_dims* dims, const void* u, const void* w_router, const void* w_experts,
    const float* dB_hat, const float* dX_hat, const float* dC_mix, float* du, float* dW_router,
    float* dW_experts, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * swimba_expert_project_mix_backward without recomputing the forward: the
 * routing, the weighted streams and the bucketing come from the forward
 * calls (the reserve-space pattern of training libraries). Results are
 * bitwise those of swimba_expert_project_mix_backward on the same inputs.
 *   topk_idx, topk_w, logits   the outputs of swimba_route_topk for u (logits
 *                              is then required)
 *   B_hat       the B_hat output of swimba_expert_project_mix for that routing
 *   fwd_ws      the workspace of that swimba_expert_project_mix call, not
 *               written since (it holds the expert-sorted pair lists and the
 *               per-slot C parts); fwd_ws_bytes as passed to it
 *   ws          workspace of swimba_workspace_size(dims, SWIMBA_CALL_PROJECT_BACKWARD_SAVED)
 * Every other argument, shape and error as for
 * swimba_expert_project_mix_backward.
 */
swimba_status swimba_expert_project_mix_backward_saved(
    const swimba_dims* dims, const void* u, const void* w_router, const void* w_experts,
    const int32_t* topk_idx, const float* topk_w, const float* logits, const void* B_hat,
    const void* fwd_ws, size_t fwd_ws_bytes, const float* dB_hat, const float* dX_hat,
    const float* dC_mix, float* du, float* dW_router, float* dW_experts, void* ws,
    size_t ws_bytes, hipStream_t stream);

/*
 * MoE over separated SSMs, the design Swimba is compared against
 * (papernotes.org notes, research background and motivation: one state
 * trajectory per expert, each expert's recursion advanced at every step, so
 * state memory and recurrence work grow with E; Method, key design 2,
 * Theorem 3.4: the output is the routing-weighted sum of the experts'
 * readouts of their own states). With the same router and expert
 * projections as the Swimba calls, for every expert e and head h:
 *   h^(e)_t = a_h h^(e)_{t-1} + [e in K_t] B^(e)_t X^(e)_t^T     (N x P, fp32)
 *   y_t     = sum_{e in K_t} pi_{t,e} C^(e)_t^T h^(e)_t
 * (an unselected expert injects nothing; its state still decays). Solved as
 * Bt * E chunked scans of k = 1 over per-expert streams (zeros where the
 * expert is not selected) in the workspace, whose fp32 outputs are summed
 * over the experts in order.
 *   u, w_router, w_experts   as for swimba_route_topk / swimba_expert_project_mix
 *   a         [H] float32
 *   h_init    [Bt, E, H, N, P] float32, or NULL for zeros
 *   y         [M, H, P] dtype out
 *   h_final   [Bt, E, H, N, P] float32 out, or NULL (may alias h_init)
 *   topk_idx  [M, k] int32 out, or NULL
 *   ws        workspace of swimba_workspace_size(dims, SWIMBA_CALL_SEPARATED)
 * Shapes and errors as for the Swimba calls; the per-expert scans take
 * dims.chunk, and the size limits of the scan apply to each trajectory.
 */
swimba_status swimba_separated_forward(const swimba_dims* dims, const void* u,
                                       const void* w_router, const void* w_experts,
                                       const float* a, const float* h_init, void* y,
                                       float* h_final, int32_t* topk_idx, void* ws,
                                       size_t ws_bytes, hipStream_t stream);

/*
 * Per-kernel timing with HIP events, for measurement only. While enabled,
 * every kernel the library launches is bracketed by two events recorded on
 * its stream. swimba_profile_report() waits for the recorded events, writes a
 * NUL-terminated JSON object {"kernel": {"launches": n, "ms": total}, ...}
 * into `buf` (host memory, `cap` bytes) and clears the records. It returns the
 * length written, or a negative swimba_status.
 */
swimba_status swimba_profile_enable(int32_t on);
int32_t swimba_profile_report(char* buf, size_t cap);
/* Restrict the timing to kernels of these names (host string, copied: one
 * name or several separated by commas); NULL or "" records every kernel.
 * Decode-step kernels carry the prefix "decode_". */
swimba_status swimba_profile_select(const char* kernel);

#ifdef __cplusplus
}
#endif

#endif /* SWIMBA_H */
