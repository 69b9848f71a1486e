/*
 * moe.h -- C ABI of one sparse mixture-of-experts layer on an MI355X (gfx950).
 *
 * The layer is the one the Strata pages describe (pyshine source tour,
 * "Understanding the Architecture"): a router scores every expert of a large
 * pool for a token, the top experts ("the router names ten experts per
 * token") run their SwiGLU MLPs, and a device-side combine sums the expert
 * outputs weighted by the router weights ("The expert handoff is a verified
 * contract": the expert side never applies the router weight, the combine
 * does).  Decode at batch 1 is a bandwidth-bound GEMV (hexlives dispatch, the
 * archived tensor-core experiment); verify windows and prefill chunks
 * ("Guess, then check" and "Prompts are read in batched pieces") run several
 * tokens through the same layer, grouped by expert.
 *
 * Conventions shared by every call:
 *  - All data pointers are DEVICE pointers except `desc`, `out`, `bytes` and
 *    `code` arguments, which are host pointers.  `stream` is a hipStream_t
 *    passed as void* (NULL = the null stream).
 *  - The caller owns every buffer it passes (weights, activations, outputs,
 *    workspace) and keeps the weights alive and unchanged while the layer
 *    exists.  The library never frees caller memory.
 *  - moe_route / moe_expert_decode / moe_grouped_forward only enqueue work on
 *    `stream`: no allocation, no host synchronisation, no device-to-host read.
 *    They can therefore be captured into a HIP graph, and their per-call
 *    values live in caller-owned fixed-address buffers (the pages' per-layer
 *    captured graphs fed through fixed-address device buffers, "One driver
 *    composes one token").  Two calls may run concurrently on different
 *    streams if each has its own workspace and outputs.
 *  - Faults that the host can detect return a negative moe_status before any
 *    work is enqueued and print nothing (a wrong expert geometry is refused
 *    rather than mis-indexed, as the handoff contract demands).  Faults only
 *    the device can see (a caller-supplied expert index out of range or
 *    repeated within a token, a non-finite router logit) set a sticky flag in
 *    the layer, make the affected token's output NaN, and are read back with
 *    moe_device_error.
 *  - T = 0 returns MOE_OK without enqueuing anything.
 *
 * Results:
 *  - idx   int32 [T][k]: the k experts with the largest logits
 *          z_e = sum_h x_h R[h][e] + b_e, ordered by (z descending, expert
 *          index ascending); z is the exact value rounded once to binary64,
 *          so ties -- and only ties -- go to the lower index.
 *  - gates fp32 [T][k]: softmax over the k selected logits.
 *  - out   fp32 [T][H]: sum_j gates[j] * D_e (silu(G_e x) * (U_e x)), e = idx[j],
 *          accumulated in fp32 (intermediate h kept in fp32).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_E_NULL = -1,        /* a required pointer is NULL */
  MOE_E_GEOMETRY = -2,    /* shapes inconsistent or unsupported */
  MOE_E_DTYPE = -3,       /* unsupported dtype or dtype combination */
  MOE_E_ALIGN = -4,       /* a device pointer is not 16-byte aligned */
  MOE_E_WORKSPACE = -5,   /* workspace NULL or smaller than moe_workspace_bytes */
  MOE_E_RANGE = -6,       /* T outside [0, max_tokens], or bad flags */
  MOE_E_HIP = -7,         /* the HIP runtime reported an error */
  MOE_E_DEVICE_FLAG = -8  /* a device-side fault was recorded (moe_device_error) */
} moe_status;

typedef enum {
  MOE_F32 = 0,            /* IEEE binary32 */
  MOE_BF16 = 1,           /* bfloat16 (upper half of a binary32) */
  MOE_Q4B32 = 2           /* 4-bit symmetric blocks, see below */
} moe_dtype;

/*
 * MOE_Q4B32 storage (expert weights only): each weight row is split into
 * blocks of 32 consecutive elements along the row's reduction dimension (H
 * for gate/up rows, I for down rows).  Element value = (nibble - 8) * d, with
 * d the block's fp16 scale.  Byte j of a row holds element 2j in its low
 * nibble and element 2j+1 in its high nibble.  Scales are a separate fp16
 * array [rows][K/32].  Nibble value 0 (q = -8) is decoded like any other.
 */

typedef enum {
  MOE_ROUTER_HE = 0,      /* router_w is the H x E matrix, row-major [H][E] */
  MOE_ROUTER_EH = 1       /* router_w is stored expert-major [E][H] (its transpose) */
} moe_router_layout;

/* desc.flags */
#define MOE_LAYER_FORCE_EXACT_REFINE 1u  /* debug: every near-tie logit goes through
                                            the slow integer accumulator */

typedef struct {
  int32_t hidden;         /* H: multiple of 8 (of 32 for MOE_Q4B32), 8 <= H <= 8192 */
  int32_t n_experts;      /* E: 1 <= E <= 1<<20 */
  int32_t top_k;          /* k: 1 <= k <= min(E, 32) */
  int32_t inter;          /* I: multiple of 8 (of 32 for MOE_Q4B32), 8 <= I <= 4096 */
  int32_t max_tokens;     /* T_max for one call: 1 <= T_max <= 65536 */
  int32_t act_dtype;      /* moe_dtype of x and of the router: MOE_F32 or MOE_BF16 */
  int32_t expert_dtype;   /* MOE_F32 (needs act MOE_F32), MOE_BF16 or MOE_Q4B32 */
  int32_t router_layout;  /* moe_router_layout */
  uint32_t flags;         /* MOE_LAYER_* bits */
  const void* router_w;   /* act_dtype, [H][E] or [E][H] per router_layout */
  const float* router_bias; /* fp32 [E], or NULL for no bias */
  const void* w_gate;     /* [E][I][H]: gate row i of expert e is contiguous along H */
  const void* w_up;       /* [E][I][H] */
  const void* w_down;     /* [E][H][I]: down row o of expert e is contiguous along I */
  const uint16_t* s_gate; /* MOE_Q4B32: fp16 scales [E][I][H/32]; else NULL */
  const uint16_t* s_up;   /* MOE_Q4B32: fp16 scales [E][I][H/32]; else NULL */
  const uint16_t* s_down; /* MOE_Q4B32: fp16 scales [E][H][I/32]; else NULL */
} moe_layer_desc;

typedef struct moe_layer moe_layer;   /* opaque; immutable after creation */

/* Validate `desc` and build a layer.  The only call that allocates device
 * memory (an expert-major router copy when router_layout is MOE_ROUTER_HE,
 * the per-expert router row norms used to bound rounding errors, the sticky
 * device-error word) and the only one that synchronises `stream`.  On error
 * *out is set to NULL. */
moe_status moe_layer_create(const moe_layer_desc* desc, void* stream, moe_layer** out);

/* Free what moe_layer_create allocated.  NULL is accepted.  The caller must
 * make sure no enqueued call still uses the layer. */
moe_status moe_layer_destroy(moe_layer* layer);

/* Device workspace, in bytes, that one call with T tokens needs (the same
 * figure serves moe_route, moe_expert_decode and moe_grouped_forward). */
moe_status moe_workspace_bytes(const moe_layer* layer, int32_t T, size_t* bytes);

/* Router + exact top-k + softmax gates for T tokens.
 *   x      [T][H] act_dtype (16-byte aligned)
 *   idx    int32 [T][k] out;  gates fp32 [T][k] out
 *   ws     device workspace of >= moe_workspace_bytes(T) bytes, 256-byte aligned */
moe_status moe_route(const moe_layer* layer, const void* x, int32_t T,
                     int32_t* idx, float* gates,
                     void* ws, size_t ws_bytes, void* stream);

/* The router step alone: z[t][e] ~ sum_h x[t][h] R[h][e] + b[e] as binary64
 * [T][E], accumulated in exactly the order that moe_route uses.  T = 1 (and
 * f32 x, or H not a multiple of 32): binary32 chains of 8 products per
 * 16-byte chunk (bf16 dot products when T > 1), then binary64 for the chain
 * sums, the wave reduction and the bias.  bf16 x with H a multiple of 32:
 * 2 <= T < 16 runs 16x16x32 MFMA tiles whose binary32 results (32 products
 * each) are added into binary64 one by one; 16 <= T < 512 runs a GEMM whose
 * binary32 accumulators are added into binary64 after every 128 of H;
 * T >= 512 runs 256x256 GEMM tiles whose binary32 accumulators run over all
 * of H before the binary64 bias addition (moe_route then keeps these logits
 * in binary32: one more rounding, covered by a 2^-24 |z| relative term).
 * With c = ceil(H / 512):
 *   |z - z_exact| <= (g(d32, 2^-23) + g(d64, 2^-52)) ||x_t||_2 max_e ||R_e||_2
 *                    + (d32 + H) 2^-125 + d64 2^-1021 + 2^-52 |z|,
 *   g(n, u) = n u / (1 - n u);  vector path: d32 = 7 (8 when T > 1),
 *   d64 = log2(c) + 7;  16x16 tiles: d32 = 33, d64 = ceil(H / 128) + 4;
 *   GEMM: d32 = 136, d64 = ceil(H / 128) + 1;  256x256 GEMM: d32 = 17 H / 16,
 *   d64 = 1.
 * moe_route recomputes exactly the logits this bound leaves undecided.
 * Useful to inspect router scores and to time the step that dominates
 * batch-1 decode.
 *   x [T][H] act_dtype; z f64 [T][E] out (8-byte aligned); ws as for moe_route. */
moe_status moe_router_logits(const moe_layer* layer, const void* x, int32_t T, double* z,
                             void* ws, size_t ws_bytes, void* stream);

/* Experts of one token: out[H] = sum_j gates[j] * expert_{idx[j]}(x).
 *   x [1][H] act_dtype; idx int32 [k]; gates fp32 [k]; out fp32 [H].
 * idx/gates normally come from moe_route; any values are accepted (the
 * gates are used as given), and bad indices raise the device flag. */
moe_status moe_expert_decode(const moe_layer* layer, const void* x,
                             const int32_t* idx, const float* gates, float* out,
                             void* ws, size_t ws_bytes, void* stream);

#define MOE_ROUTE_INTERNAL 0u  /* route inside the call; write idx/gates if non-NULL */
#define MOE_ROUTE_GIVEN    1u  /* read caller idx/gates [T][k] instead of routing */

/* The whole layer for T tokens: route (or take the given routing), group the
 * T*k token-expert pairs by expert, run each active expert once over its
 * tokens, and un-permute with the weighted combine.  out fp32 [T][H].
 * idx and gates are identical to those of moe_route on the same T tokens;
 * row t of out equals moe_expert_decode of x[t] with that routing within
 * fp32 accumulation error (bit for bit at T = 1, where the selection runs
 * fused with the gate/up projections). */
moe_status moe_grouped_forward(const moe_layer* layer, const void* x, int32_t T,
                               int32_t* idx, float* gates, uint32_t flags,
                               float* out, void* ws, size_t ws_bytes, void* stream);

/* Synchronise `stream`, return the sticky device-fault bits in *code (0 when
 * clean: 1 = expert index out of range, 2 = expert repeated within a token,
 * 4 = non-finite router logit, 8 = internal range check) and clear them.
 * Returns MOE_E_DEVICE_FLAG when *code != 0. */
moe_status moe_device_error(const moe_layer* layer, void* stream, int32_t* code);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* Detail of the last failing call on this host thread ("" if none). */
const char* moe_last_error_message(void);

/* ABI version of this header (bumped on incompatible changes). */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
