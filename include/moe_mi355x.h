/*
 * moe_mi355x.h -- C ABI of a deterministic, batch-invariant routed
 * mixture-of-experts layer for AMD Instinct MI355X (gfx950).
 *
 * The layer is the one described on the RL-Kernel pull request 557 page
 * (Qwen3-Next EP4 distributed logprob parity), in the commit message of its
 * stack entry "MoE route/combine contract with a batch-invariant grouped
 * expert GEMM", with the model shape of the SkyRL pull request 2513 page
 * (section "What": 512 routed experts, top-10, a shared expert):
 *
 *   route    FP32 router projection, softmax, stable descending top-k with
 *            ties to the lower expert id, FP32 renormalisation of the
 *            selected gates                       (contract, Routing bullet)
 *   permute  counting sort of the token-routes by expert    (page "What":
 *            dispatch is a local selection of each expert's routes)
 *   ffn      per-route gate_up and down projections with one fixed tile
 *            configuration, no gate multiply and no sum inside, exactly one
 *            writer per (token, route) row              (Experts bullet)
 *   combine  the route terms summed in FP32 in route order, one cast to
 *            BF16, no atomics                          (Combine bullet)
 *   backward per-expert weight gradients into dense buffers, each token's
 *            input gradient summed over its routes in ascending expert id
 *                                                        (Backward bullet)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Dimensions: T tokens, H hidden, E experts, K routes per token, I expert
 *    intermediate size, Is shared-expert intermediate size (0 = no shared
 *    expert).  R = T*K route rows.  Route id r = t*K + k (slot k of token t).
 *  - bf16 tensors are passed as uint16_t bit patterns.  All tensors are
 *    dense, row-major, in device memory, 16-byte aligned.
 *  - Ownership: the caller owns every buffer.  The library never allocates,
 *    frees or keeps a pointer past the call, and never synchronises the
 *    stream.  All work is enqueued on `stream` in call order.
 *  - Outputs are fully overwritten; nothing accumulates into caller memory.
 *  - Errors: every call validates its arguments on the host before it
 *    enqueues anything; on failure it returns a non-zero status and has
 *    enqueued nothing (fail closed).  Bad data found on the device (a
 *    caller-supplied expert id out of range or repeated within a token) sets
 *    an error word in the workspace, which each moe_permute, moe_forward,
 *    moe_backward and moe_backward_lora overwrites; caller-supplied
 *    expert_offsets that are not a partition of [0, T*K) (moe_grouped_ffn,
 *    moe_grouped_ffn_lora, moe_backward, moe_backward_lora) set it too and
 *    the call then computes nothing; moe_last_device_error() reads it.
 *  - Supported sizes: E % 64 == 0 and 64 <= E <= 1024; 1 <= K <= 16 and
 *    K <= E; H % 256 == 0, 256 <= H <= 16384; I % 128 == 0, 128 <= I <= 4096;
 *    Is == 0 or the same rule as I; 0 <= T and T*K < 2^31.  T == 0 returns
 *    MOE_OK and enqueues nothing.
 *  - Determinism: every output is a pure function of the inputs, identical
 *    bit for bit across runs, streams and batch compositions: a token's
 *    routes, gates, route rows, output and input gradient do not depend on
 *    the other tokens in the batch or on its position.  Weight gradients are
 *    sums over the batch: deterministic, but naturally batch-dependent.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

enum moe_status {
  MOE_OK = 0,
  MOE_E_NULL = 1,        /* a required pointer is NULL                         */
  MOE_E_SHAPE = 2,       /* a dimension is out of the supported range          */
  MOE_E_UNSUPPORTED = 3, /* a valid but unsupported combination                */
  MOE_E_ALIGN = 4,       /* a pointer is not 16-byte aligned                   */
  MOE_E_WORKSPACE = 5,   /* workspace NULL or smaller than moe_workspace_bytes */
  MOE_E_DEVICE = 6,      /* current device is not gfx950, or device data error */
  MOE_E_LAUNCH = 7,      /* a kernel launch failed                             */
  MOE_E_ALIAS = 8        /* an output overlaps an input or another output      */
};

/* operation ids for moe_workspace_bytes */
enum moe_op {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_FFN = 2,
  MOE_OP_FORWARD = 3,
  MOE_OP_BACKWARD = 4,
  MOE_OP_FORWARD_LORA = 5,
  MOE_OP_BACKWARD_LORA = 6
};

typedef struct moe_dims {
  int64_t tokens;       /* T */
  int32_t hidden;       /* H */
  int32_t experts;      /* E */
  int32_t top_k;        /* K */
  int32_t inter;        /* I  */
  int32_t shared_inter; /* Is (0: no shared expert) */
} moe_dims;

typedef struct moe_weights {
  const float* w_router;    /* [E][H] fp32                                   */
  const float* router_bias; /* [E] fp32 added to the logits, or NULL          */
  const uint16_t* w13;      /* [E][2I][H] bf16: rows 0..I-1 gate, I..2I-1 up  */
  const uint16_t* w2;       /* [E][H][I] bf16                                 */
  const uint16_t* ws13;     /* [2Is][H] bf16 shared gate/up (NULL iff Is==0)  */
  const uint16_t* ws2;      /* [H][Is] bf16 shared down (NULL iff Is==0)      */
  const uint16_t* w_sgate;  /* [H] bf16 shared-expert gate (NULL iff Is==0)   */
  const uint16_t* w_router_planes; /* [3][E][H] bf16: w_router's exact split
                         (moe_split_router), made once and reused by every
                         call, or NULL: each call splits w_router itself.  If
                         given it must be moe_split_router's result for this
                         w_router (it is what the router multiplies). */
} moe_weights;

typedef struct moe_routes {
  int32_t* topk_idx;       /* [T][K] expert id of slot k, slot 0 the largest */
  float* topk_gate;        /* [T][K] renormalised gate of slot k             */
  float* logits;           /* [T][E] fp32 router logits, or NULL             */
  int32_t* expert_offsets; /* [E+1] start of expert e's segment; [E] = R     */
  int32_t* sorted_route;   /* [R] route ids sorted by (expert, route id)     */
  int32_t* route_pos;      /* [R] inverse: sorted_route[route_pos[r]] == r   */
} moe_routes;

typedef struct moe_saved {
  float* y;           /* [R][H] fp32 expert output of route r (row r=t*K+k)   */
  float* gu;          /* [R][2I] fp32 gate|up pre-activations, row = sorted
                         position p (NULL: not saved, forward-only)          */
  float* shared_y;    /* [T][H] fp32 shared-expert output (Is>0)             */
  float* shared_gate; /* [T] fp32 sigmoid(w_sgate . x) (Is>0)                */
  float* shared_gu;   /* [T][2Is] fp32 shared gate|up (NULL: not saved)      */
} moe_saved;

typedef struct moe_grads {
  float* d_w_router; /* [E][H]      */
  float* d_w13;      /* [E][2I][H]  */
  float* d_w2;       /* [E][H][I]   */
  float* d_ws13;     /* [2Is][H]    (Is>0) */
  float* d_ws2;      /* [H][Is]     (Is>0) */
  float* d_w_sgate;  /* [H]         (Is>0) */
} moe_grads;

/* MOE_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* moe_status_str(int status);

/* Bytes of device workspace the operation `op` (enum moe_op) needs for these
 * dims; 0 if the dims are invalid.  The workspace is scratch owned by the
 * caller; its contents between calls carry only the device-error word of
 * the last permutation.  Size it once per shape; a workspace sized for MOE_OP_BACKWARD also
 * serves every other operation at the same dims. */
size_t moe_workspace_bytes(const moe_dims* dims, int op);

/* Route (contract, Routing bullet).
 * x [T][H] bf16.  Writes logits (if routes->logits != NULL), topk_idx and
 * topk_gate.  The router logit l[t][e] = sum_h x[t][h] * w_router[e][h]
 * (+ router_bias[e]) is formed with exact bf16 x fp32 products (the fp32
 * weight split exactly into three bf16 parts, multiplied on the matrix
 * cores), summed in fixed 256-wide chunks in fp32 and across chunks in fp64,
 * then rounded to fp32.  Selection compares those fp32 logits (greater first, equal values
 * to the lower id); the gates are exp(l_k - l_0) / sum_j exp(l_j - l_0) over
 * the selected slots, in fp32. */
int moe_route(const moe_dims* dims, const uint16_t* x, const moe_weights* w,
              moe_routes* routes, void* ws, size_t ws_bytes, hipStream_t stream);

/* The router weight's exact split (Routing bullet: the FP32 router on bf16
 * matrix cores): planes[q][e][h], q = 0, 1, 2, with hi = bf16(w), mid =
 * bf16(w - hi), lo = bf16(w - hi - mid), round to nearest even, so that
 * hi + mid + lo == w exactly for every finite fp32 w.  The router is constant
 * across calls, so a caller splits it once and passes the planes as
 * moe_weights.w_router_planes; without them every routing call makes this
 * split in its workspace first (one more kernel).  Uses dims' E and H only;
 * no workspace.  Errors: MOE_E_NULL, MOE_E_SHAPE, MOE_E_ALIGN, MOE_E_ALIAS
 * (planes overlapping w_router), MOE_E_DEVICE. */
int moe_split_router(const moe_dims* dims, const float* w_router, uint16_t* planes,
                     hipStream_t stream);

/* Permute (page "What": local selection of each expert's routes).
 * Reads routes->topk_idx (from moe_route, or supplied by the caller, e.g.
 * replayed routing) and writes expert_offsets, sorted_route and route_pos:
 * a stable counting sort of route ids by expert (ascending route id inside
 * each expert's segment).  Out-of-range or repeated ids within a token set
 * the workspace's device-error word (cleared otherwise) and leave the
 * permutation unspecified. */
int moe_permute(const moe_dims* dims, moe_routes* routes, void* ws, size_t ws_bytes,
                hipStream_t stream);

/* Grouped expert FFN (contract, Experts bullet).
 * For each route r of expert e: gu = W13_e x[t] (fp32 accumulation of exact
 * bf16 products, fixed K order), act = silu(gate) * up in fp32, passed to
 * the down projection as a bf16 hi/lo pair, y = W2_e act accumulated in fp32
 * and written to saved->y row r; one writer per row, no gate multiply.  The
 * shared expert (Is > 0) runs through the same kernels on all T tokens and
 * writes saved->shared_y, and saved->shared_gate = sigmoid(w_sgate . x).
 * Needs the permutation of moe_permute.  saved->gu / shared_gu are written
 * when non-NULL (needed by moe_backward). */
int moe_grouped_ffn(const moe_dims* dims, const uint16_t* x, const moe_weights* w,
                    const moe_routes* routes, moe_saved* saved, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* Combine (contract, Combine bullet).
 * out[t] = fma chain over k = 0..K-1 of topk_gate[t][k] * y[t*K+k] starting
 * from +0, then one more fma with shared_gate[t] * shared_y[t] (Is > 0),
 * all in fp32; out_f32 gets that value, out_bf16 its round-to-nearest-even
 * bf16.  Either output may be NULL, not both.  No atomics. */
int moe_combine(const moe_dims* dims, const moe_routes* routes, const moe_saved* saved,
                float* out_f32, uint16_t* out_bf16, hipStream_t stream);

/* Whole forward: route, permute, grouped FFN, combine, in that order on
 * `stream`.  routes->logits may be NULL (the logits are then not stored). */
int moe_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* x,
                moe_routes* routes, moe_saved* saved, float* out_f32, uint16_t* out_bf16,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward (contract, Backward bullet).
 * Inputs: the forward's x, routes and saved tensors (saved->gu, and
 * saved->shared_gu and saved->shared_gate when Is > 0, must have been
 * written; saved->y and saved->shared_y are not read and may be NULL),
 * d_out [T][H] bf16.
 * Outputs: d_x_f32 [T][H] (and its bf16 rounding in d_x_bf16 if non-NULL)
 * and every weight gradient in `grads` (fp32, overwritten).
 *   dg[t][k] = <d_out[t], y[t*K+k]>, formed as the equal sum over the
 *              intermediate size <W2_e^T d_out[t], act>, in fp64 from the
 *              fp32 GEMM product and the fp32 activation recomputed from
 *              saved->gu, in a fixed per-route order (the shared gate's
 *              <d_out, shared_y> likewise)
 *   dl = g * (dg - sum_j g_j dg_j)     (softmax backward over selected slots)
 *   route r: dy = g * d_out[t]; dact = dy W2_e; SwiGLU backward -> dgu;
 *            dx_r = dgu W13_e; dW2_e = sum_r dy^T act; dW13_e = sum_r dgu^T x
 *   shared:  dz = <d_out, shared_y> sg (1 - sg); dw_sgate = sum_t dz x;
 *            same expert backward with dy = sg * d_out
 *   router:  d_w_router[e] = sum_t dl[t][e] x[t];  dx_router = sum_k dl W_r
 *   d_x[t] = ((sum of dx_r over its routes in ascending expert id) +
 *            dx_shared) + dz * w_sgate + dx_router, in that order, fp32.
 * Precision: the weight-gradient GEMMs take their fp32 operands (dgu,
 * g * act) exactly as three bf16 planes; products of bf16 values are exact
 * and accumulate in fp32.  Weight-gradient sums run over routes (tokens) in
 * ascending order; no atomics anywhere. */
int moe_backward(const moe_dims* dims, const moe_weights* w, const uint16_t* x,
                 const moe_routes* routes, const moe_saved* saved, const uint16_t* d_out,
                 float* d_x_f32, uint16_t* d_x_bf16, moe_grads* grads, void* ws,
                 size_t ws_bytes, hipStream_t stream);

/* Streams and events of the caller that let moe_backward_side run its
 * independent weight-gradient GEMMs beside the input-gradient GEMM.  The
 * caller creates and owns all of them (streams of default priority, events
 * preferably with hipEventDisableTiming); the library only records and
 * waits on them, so concurrent calls must not share them. */
typedef struct {
  hipStream_t side[2]; /* two streams other than the call's and each other */
  hipEvent_t fork;     /* recorded on the call's stream, waited for by both */
  hipEvent_t join[2];  /* recorded on side[i], waited for by the call's stream */
} moe_side_streams;

/* Backward (contract, Backward bullet: the operation of moe_backward) with
 * its three independent grouped GEMMs on three streams:
 * dW13 on side[0] and dW2 on side[1], from the point where the activation
 * gradients exist (`fork`), dx and the kernels after it on `stream`, which
 * then waits for both side streams (`join`), so work enqueued on `stream`
 * after this call sees every output.  The store-bound weight gradients then
 * share the CUs with the load-bound dx GEMM.  Results are bit for bit those
 * of moe_backward (the same kernels on the same data).  Errors as
 * moe_backward, plus MOE_E_NULL for a missing stream or event and
 * MOE_E_ALIAS for streams or events that are not distinct. */
int moe_backward_side(const moe_dims* dims, const moe_weights* w, const uint16_t* x,
                      const moe_routes* routes, const moe_saved* saved, const uint16_t* d_out,
                      float* d_x_f32, uint16_t* d_x_bf16, moe_grads* grads, void* ws, size_t ws_bytes,
                      hipStream_t stream, const moe_side_streams* side);

/* Whole forward (contract, Routing, Experts and Combine bullets; the shared
 * expert of the SkyRL pull request 2513 page's What section: the operation
 * of moe_forward) with the shared expert on side[0]: its two GEMMs, which do
 * not depend on the routing, run from the call's start (`fork`) on lists of
 * their own, beside the router, top-k, permutation and routed GEMMs on
 * `stream`; `stream` waits for them (`join[0]`) before the combine.  The
 * routed GEMMs' lists then hold routed tiles only.  Results are bit for bit
 * those of moe_forward.  side[1] and join[1] are not used (validated as in
 * moe_backward_side).  Without a shared expert it is moe_forward.  Errors as
 * moe_forward and moe_backward_side. */
int moe_forward_side(const moe_dims* dims, const moe_weights* w, const uint16_t* x,
                     moe_routes* routes, moe_saved* saved, float* out_f32, uint16_t* out_bf16,
                     void* ws, size_t ws_bytes, hipStream_t stream, const moe_side_streams* side);

/* Block-scaled FP8 expert weights (OCP MX format, the E4M3 element type).
 * Every 32 consecutive elements of a weight row along its contraction axis
 * (H for W13 / Ws13, I for W2 / Ws2) share one E8M0 scale code s, value
 * 2^(s - 127); an element is an E4M3 code (1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits; code 0x7F / 0xFF is NaN).  The weight this represents
 * is code value x 2^(s - 127), exactly: an E4M3 value has at most 4
 * significant bits, so every represented weight in bf16 range is a bf16.
 * Layouts are those of moe_weights with one byte per element; the scale
 * arrays have one byte per 32 elements.  Scale code 255 (NaN) is not
 * allowed.  Router, bias and shared gate are as in moe_weights. */
typedef struct {
  const float* w_router;    /* [E][H] fp32 */
  const float* router_bias; /* [E] fp32 or NULL */
  const uint8_t* w13_q;     /* [E][2I][H] E4M3 */
  const uint8_t* w13_s;     /* [E][2I][H/32] E8M0 */
  const uint8_t* w2_q;      /* [E][H][I] E4M3 */
  const uint8_t* w2_s;      /* [E][H][I/32] E8M0 */
  const uint8_t* ws13_q;    /* [2Is][H] (NULL iff Is == 0) */
  const uint8_t* ws13_s;    /* [2Is][H/32] */
  const uint8_t* ws2_q;     /* [H][Is] */
  const uint8_t* ws2_s;     /* [H][Is/32] */
  const uint16_t* w_sgate;  /* [H] bf16 (NULL iff Is == 0) */
  const uint16_t* w_router_planes; /* [3][E][H] bf16 or NULL, as in moe_weights */
} moe_weights_mx;

/* Forward with block-scaled FP8 expert weights (the MXFP8 item of the
 * SkyRL pull request 2513 page's progress list, Stage 3: performance and
 * quantization, follow-up).
 * Same contract, kernels and per-element arithmetic as moe_forward with
 * each expert weight replaced by its represented value: the expert GEMMs
 * expand every 16 codes to bf16 with the gfx950 scaled conversion as they
 * stage them, so for equal represented weights the results are bit for bit
 * those of moe_forward.  Reads about half of moe_forward's weight bytes.
 * Same errors as moe_forward. */
int moe_forward_mx(const moe_dims* dims, const moe_weights_mx* w, const uint16_t* x,
                   moe_routes* routes, moe_saved* saved, float* out_f32, uint16_t* out_bf16,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* LoRA adapters of the routed experts (ROLL pull request 502 page,
 * Qwen3.8-Flash-Next adapter: grouped expert adapters of rank r // top_k,
 * "What this changes"; the adapters' shrink with a single K partition, no
 * fp32 atomics, opening summary).  Expert e's two projections get the
 * update scale * B (A v) (LoRA, Hu et al., section 4.1, with the caller's
 * scale, e.g. alpha / r):
 *   gate/up:  gu_r += scale * B13_e (A13_e x_t)
 *   down:     y_r  += scale * B2_e (A2_e act_r)
 * All matrices bf16, row-major, caller-owned, 16-byte aligned:
 *   a13 [E][rank][H], b13 [E][2I][rank], a2 [E][rank][I], b2 [E][H][rank].
 * 1 <= rank <= 16.  The shared expert and the router have no adapter. */
typedef struct {
  int32_t rank;
  float scale;
  const uint16_t* a13;
  const uint16_t* b13;
  const uint16_t* a2;
  const uint16_t* b2;
} moe_lora;

/* Forward of the layer whose routed experts carry LoRA adapters.  Kernels
 * and per-element arithmetic of moe_forward, plus two shrink kernels and
 * the expand inside the grouped GEMMs' epilogues:
 *   z[p][j] = sum_k A_e[j][k] v_p[k] (16x16x32 bf16 MFMAs over ascending
 *            32-wide K steps, fp32 accumulation, one wave per 32 rows and
 *            the whole contraction), v_p = x_t for the gate/up adapter, act_r
 *            (its bf16 hi + lo, two passes) for down; kept as a bf16 pair
 *            z_hi + z_lo;
 *   t = z_hi B^T + z_lo B^T (two bf16 MFMAs, fp32 accumulation, over 16
 *            zero-padded rank columns), then gate/up (and y) = fma(scale, t,
 *            GEMM accumulator), before the SwiGLU (and before y is stored).
 * So every route row is a function of its own data only (batch invariant,
 * deterministic, no atomics).  saved->gu, if given, receives the gate/up
 * values with the update (moe_backward_lora needs them).  Workspace:
 * moe_workspace_bytes(dims, MOE_OP_FORWARD_LORA).  Errors as moe_forward,
 * plus MOE_E_NULL for a missing adapter matrix and MOE_E_SHAPE for a rank
 * outside 1..16. */
int moe_forward_lora(const moe_dims* dims, const moe_weights* w, const moe_lora* lora,
                     const uint16_t* x, moe_routes* routes, moe_saved* saved, float* out_f32,
                     uint16_t* out_bf16, void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouped FFN stage of moe_forward_lora on a caller-made permutation, as
 * moe_grouped_ffn is to moe_forward (routing replay: moe_permute on
 * replayed topk_idx, then this, then moe_combine give moe_forward_lora's
 * bits for the same routes).  Workspace: moe_workspace_bytes(dims,
 * MOE_OP_FORWARD_LORA).  Errors as moe_grouped_ffn and moe_forward_lora. */
int moe_grouped_ffn_lora(const moe_dims* dims, const uint16_t* x, const moe_weights* w,
                         const moe_lora* lora, const moe_routes* routes, moe_saved* saved, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* Gradients of the routed experts' adapters, fp32, caller-owned, 16-byte
 * aligned, overwritten, in the adapters' layouts:
 *   d_a13 [E][rank][H], d_b13 [E][2I][rank], d_a2 [E][rank][I], d_b2 [E][H][rank].
 * An expert with no routes gets zeros. */
typedef struct {
  float* d_a13;
  float* d_b13;
  float* d_a2;
  float* d_b2;
} moe_lora_grads;

/* Backward of moe_forward_lora: the adapters are trained (ROLL pull request
 * 502 page, opening summary: LoRA SFT, RL and OPD over the grouped expert
 * adapters of the "What this changes" rank bullet).  Inputs and outputs of
 * moe_backward, with saved->gu from moe_forward_lora (gate/up values with
 * the update), plus the adapters and their gradients.  With s = scale and
 * route r of expert e (token t, gate g, dy = g d_out[t]), by the chain rule
 * through gu += s B13 (A13 x) and y += s B2 (A2 act):
 *   v2   = B2^T dy / g = B2^T d_out[t]      (shrink, before the dact GEMM)
 *   dact = dy W2_e + s g A2^T v2            (LoRA term added to the GEMM
 *          product before the SwiGLU backward; dg[t][k] likewise uses
 *          <W2_e^T d_out[t] + s A2^T v2, act>, the route's y with the update)
 *   u13  = B13^T dgu;   dx_r = dgu W13_e + s A13^T u13
 *   dA13_e = s sum_r u13 x^T      dB13_e = s sum_r dgu (A13 x)^T
 *   dA2_e  = s sum_r g v2 act^T   dB2_e  = s sum_r d_out[t] (A2 g act)^T
 * the base weight gradients and everything else as in moe_backward.  The
 * shrinks (v2, u13, A13 x, A2 (g act)) are those of moe_forward_lora's
 * shrink kernel (fp32 on the matrix cores, kept as bf16 hi + lo pairs; dgu
 * and g act enter them as their first two bf16 planes, 16 significant
 * bits); the expand terms run on the matrix cores in the grouped GEMMs'
 * epilogues as in the forward; each adapter-gradient sum runs over the
 * expert's routes in sorted order in fp32 (four contiguous quarters of the
 * routes summed separately, then added in quarter order), with dgu and
 * g act exact (three planes).  No atomics; results are deterministic.  Workspace:
 * moe_workspace_bytes(dims, MOE_OP_BACKWARD_LORA).  Errors as moe_backward,
 * plus MOE_E_NULL for a missing adapter, gradient struct or adapter
 * gradient and MOE_E_SHAPE for a rank outside 1..16. */
int moe_backward_lora(const moe_dims* dims, const moe_weights* w, const moe_lora* lora,
                      const uint16_t* x, const moe_routes* routes, const moe_saved* saved,
                      const uint16_t* d_out, float* d_x_f32, uint16_t* d_x_bf16, moe_grads* grads,
                      moe_lora_grads* lora_grads, void* ws, size_t ws_bytes, hipStream_t stream);

/* LoRA backward (ROLL pull request 502 page, opening summary: the operation
 * of moe_backward_lora) with the base weight gradients on the side streams as in
 * moe_backward_side (the adapter gradients stay on `stream`, after dx).
 * Bit for bit moe_backward_lora.  Errors as moe_backward_lora and
 * moe_backward_side. */
int moe_backward_lora_side(const moe_dims* dims, const moe_weights* w, const moe_lora* lora,
                           const uint16_t* x, const moe_routes* routes, const moe_saved* saved,
                           const uint16_t* d_out, float* d_x_f32, uint16_t* d_x_bf16, moe_grads* grads,
                           moe_lora_grads* lora_grads, void* ws, size_t ws_bytes, hipStream_t stream,
                           const moe_side_streams* side);

/* Profiling variant of moe_forward: the same kernels in the same order on
 * `stream`, with events[i] recorded just before kernel i and events[n] after
 * the last one, n = moe_forward_kernel_count(dims).  `events` are created by
 * the caller (hipEventCreate); a NULL entry records nothing at its position
 * (so a caller can time one kernel with two events and leave the others
 * unmarked); n_events must be >= n + 1.  Results are
 * identical to moe_forward.  Kernel order (moe_forward_kernel_name gives
 * the names): router_split, router_logits, topk_gate (which also forms the
 * shared-expert gate when Is > 0), the permutation (route_sort, one kernel,
 * when experts * ceil(tokens / 32) <= 16384, else route_hist, route_scan,
 * route_scatter), ffn_up, ffn_down, combine. */
int moe_forward_profiled(const moe_dims* dims, const moe_weights* w, const uint16_t* x,
                         moe_routes* routes, moe_saved* saved, float* out_f32,
                         uint16_t* out_bf16, void* ws, size_t ws_bytes, hipEvent_t* events,
                         int n_events, hipStream_t stream);

/* Number of kernels moe_forward launches for these dims (0 if invalid). */
int moe_forward_kernel_count(const moe_dims* dims);

/* Name of kernel i (0-based, launch order) of moe_forward for these dims, a
 * static string; NULL if the dims are invalid or i is out of range. */
const char* moe_forward_kernel_name(const moe_dims* dims, int i);

/* Size of the device array that moe_forward_noalloc uses as its workspace
 * (one array per GPU, held by the library until the process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): moe_forward
 * with its workspace in a library-owned device array of
 * MOE_NOALLOC_SCRATCH_BYTES instead of a caller buffer; the caller still
 * passes every input and output.  Same kernels, arguments, results (bit for
 * bit) and errors as moe_forward, plus MOE_E_WORKSPACE when these dims need
 * a larger workspace than the array (moe_workspace_bytes(dims,
 * MOE_OP_FORWARD) > MOE_NOALLOC_SCRATCH_BYTES: at hidden 2048, 512 experts
 * top-10, intermediate 512, up to about 1550 tokens); the device's array is
 * looked up before the other arguments are checked, so without a current
 * gfx950 device it returns MOE_E_DEVICE first.  Allocates nothing and
 * calls no allocating routine; the first call on a device looks the array's
 * address up once.  All calls on one GPU share its array: calls that overlap
 * on one GPU (other streams or threads) race.  moe_last_device_error cannot
 * read this workspace; a bad caller route shows only through the outputs. */
int moe_forward_noalloc(const moe_dims* dims, const moe_weights* w, const uint16_t* x,
                        moe_routes* routes, moe_saved* saved, float* out_f32, uint16_t* out_bf16,
                        hipStream_t stream);

/* Synchronises `stream`, then returns the device error word of workspace
 * `ws` (MOE_OK or MOE_E_DEVICE) as left by the calls on that workspace
 * since the last one that overwrites it (moe_permute, moe_forward,
 * moe_backward, moe_backward_lora).
 * Debug/validation use. */
int moe_last_device_error(void* ws, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
