/*
 * moe.h -- C ABI of one sparse mixture-of-experts layer on an MI355X (gfx950).
 *
 * The layer is the one the Strata pages describe (pyshine source tour,
 * section Understanding the Architecture): a router scores every expert of a
 * large pool for a token, the ten best-scoring experts run their SwiGLU MLPs
 * (the end-to-end paragraph of that section), and a device-side combine sums
 * the expert outputs weighted by the router weights (paragraph on the expert
 * hand-off: the expert side never applies the router weight, the combine
 * does).  Decode at batch 1 is a GEMV limited by memory bandwidth (hexlives
 * dispatch, paragraph on the archived tensor-core benchmark); verify windows
 * and prefill chunks (pyshine tour, same section, the paragraphs on
 * speculative decoding and on chunked prompt reading) run several tokens
 * through the same layer, grouped by expert.
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
 *    values live in caller-owned fixed-address buffers (the pages capture one
 *    graph per layer and feed it through fixed-address device buffers: pyshine
 *    tour, Understanding the Architecture, paragraph on the engine driver).
 *    Two calls may run concurrently on different
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
#define MOE_LAYER_SCREEN_ON  2u  /* build the router screen even when E < 4096 */
#define MOE_LAYER_SCREEN_OFF 4u  /* never build it (batch-1 routing reads the bf16 router) */
#define MOE_LAYER_WINDOW_SCREEN_OFF 8u  /* verify windows (2 <= T <= 8) route on the bf16
                                           router even when the layer has the screen */

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

/* Validate `desc` and build a layer (the pages' hand-off contract refuses a
 * wrong expert geometry instead of mis-indexing it: pyshine tour,
 * Understanding the Architecture, paragraph on the expert hand-off).  The
 * only call that allocates device
 * memory (an expert-major router copy when router_layout is MOE_ROUTER_HE,
 * the per-expert router row norms used to bound rounding errors, the sticky
 * device-error word, and -- for bf16 activations, H a multiple of 32 and
 * E >= 4096 unless MOE_LAYER_SCREEN_OFF, or with MOE_LAYER_SCREEN_ON -- the
 * router screen: an int8 copy
 * of the router with a per-expert scale and residual norms, E H + 12 E
 * bytes, see moe_router_screen; for H <= 2048 and max_tokens >= 2, unless
 * MOE_LAYER_WINDOW_SCREEN_OFF, a second int8 copy in matrix-core operand
 * order for verify windows, E H bytes) and the only one that synchronises
 * `stream` (with moe_layer_set_hot_experts / moe_layer_set_host_experts).
 * Returns MOE_E_RANGE when the router weights or the bias are not finite.
 * On error *out is set to NULL. */
moe_status moe_layer_create(const moe_layer_desc* desc, void* stream, moe_layer** out);

/* Free what moe_layer_create allocated.  NULL is accepted.  The caller must
 * make sure no enqueued call still uses the layer. */
moe_status moe_layer_destroy(moe_layer* layer);

/* Device workspace, in bytes, that one call with T tokens needs (the same
 * figure serves moe_route, moe_expert_decode and moe_grouped_forward). */
moe_status moe_workspace_bytes(const moe_layer* layer, int32_t T, size_t* bytes);

/* Router + exact top-k + softmax gates for T tokens: the router names the
 * ten experts a token runs (pyshine tour, Why You Need This and Understanding
 * the Architecture, the paragraph on the routing kernel); the order is
 * decided on exact logits, ties to the lower index.
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

/* The router's int8 first pass ("screen"), which moe_route and
 * moe_grouped_forward use for T = 1 and for verify windows of 2 to 8 tokens
 * on layers that have one (windows: on the int8 matrix cores, values
 * identical to the batch-1 screen's).  The pages'
 * routing kernel scores every expert for each token (pyshine tour,
 * Understanding the Architecture, paragraph on the residency tiers); at
 * batch 1 that pass is bound by the router bytes it reads, so the screen
 * reads an int8 copy (q_e = rint(R_e / s_e), s_e = max|R_e| / 127) with the
 * hidden state in a 15-bit fixed point, and
 *   v[t][e] = s_e 2^-m sum_h q_eh X_th + b_e     (exact integer dot products),
 *   |v - z| <= bound[t][e] = ||x_t|| ||R_e - s_e q_e|| + ||delta_t|| ||s_e q_e||
 *                            + 2^-23 |v| + 2^-52 max|b| + 2^-140,
 * where z is the exact logit and delta_t the rounding of x_t to the fixed
 * point.  The routing recomputes exactly the experts whose interval reaches
 * the k-th largest lower end, so idx and gates do not depend on the screen.
 *   x [T][H] bf16; v fp32 [T][E] out; bound fp32 [T][E] out or NULL (then
 *   one kernel runs: the screen alone); ws as for moe_route.
 * Returns MOE_E_DTYPE for a layer without a screen. */
moe_status moe_router_screen(const moe_layer* layer, const void* x, int32_t T, float* v, float* bound,
                             void* ws, size_t ws_bytes, void* stream);

/* Experts of one token: out[H] = sum_j gates[j] * expert_{idx[j]}(x), the
 * gates applied once, at the combine (pyshine tour, Understanding the
 * Architecture, paragraph on the expert hand-off); the single-token expert
 * GEMVs are bandwidth-bound and run on the vector units (hexlives dispatch,
 * paragraph on the archived tensor-core benchmark).
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
 * T = 1 is a decode step, 2 <= T <= 8 a verify window of drafted tokens,
 * larger T a prefill chunk (pyshine tour, Understanding the Architecture,
 * the paragraphs on guessing then checking drafts and on reading prompts in
 * chunks).
 * idx and gates are identical to those of moe_route on the same T tokens;
 * row t of out equals moe_expert_decode of x[t] with that routing within
 * fp32 accumulation error (bit for bit at T = 1, where the selection runs
 * fused with the gate/up projections). */
moe_status moe_grouped_forward(const moe_layer* layer, const void* x, int32_t T,
                               int32_t* idx, float* gates, uint32_t flags,
                               float* out, void* ws, size_t ws_bytes, void* stream);

/* moe_grouped_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The per-call scratch lives in the
 * library's own fixed device array of 8 MiB on each GPU (held until the
 * process ends); the call allocates nothing and returns MOE_E_WORKSPACE when
 * moe_workspace_bytes(T) exceeds 8 MiB (at H = 2048, E = 24,576, k = 10,
 * I = 256 that covers decode and verify windows, T up to about 20), and
 * MOE_E_RANGE when the current device is not the layer's.  Every call on one GPU shares that array and leaves its contents
 * behind: calls that may overlap on one GPU (other streams, other host
 * threads) race and must not be issued.  Arguments and results otherwise as
 * moe_grouped_forward. */
moe_status moe_grouped_forward_noalloc(const moe_layer* layer, const void* x, int32_t T,
                                       int32_t* idx, float* gates, uint32_t flags,
                                       float* out, void* stream);

/* Faults only the device sees (the hand-off contract's refusal of bad
 * geometry, per token: pyshine tour, paragraph on the expert hand-off).
 * Synchronise `stream`, return the sticky device-fault bits in *code (0 when
 * clean: 1 = expert index out of range, 2 = expert repeated within a token,
 * 4 = non-finite router logit, 8 = internal range check) and clear them.
 * Returns MOE_E_DEVICE_FLAG when *code != 0. */
moe_status moe_device_error(const moe_layer* layer, void* stream, int32_t* code);

/* Statistics: synchronise `stream` and return in *exact_refinements how many
 * logits the layer's selections have refined exactly since it was created
 * (the integer-bin accumulation run when a logit's error interval overlaps
 * a neighbour's at the order of the k chosen experts or at the cut; see the
 * selection's certification).  Host pointer; MOE_E_NULL when it is NULL. */
moe_status moe_layer_stats(const moe_layer* layer, void* stream, uint64_t* exact_refinements);

/* ---- Hot-expert region.
 *
 * The pages keep the most-routed experts in the fastest memory and move the
 * set as the routed topics shift, using a record of how often each expert
 * is chosen (pyshine source tour, Understanding the Architecture, the
 * paragraph on three tiers and one residency table; hexlives dispatch, the
 * paragraph on the calibration step that decides which experts earn the
 * space).  Here every expert already sits in HBM, so the region is a
 * compact copy of chosen experts -- fewer DRAM pages and a footprint the
 * 256 MB Infinity Cache can hold -- which the few-token path (T <= 25
 * pairs per call: batch-1 decode and verify windows) reads instead of the
 * pool; larger calls keep reading the pool.  Results are bitwise the same
 * with or without a region. */

/* Per-expert choice counts: counts[e] += 1 (uint32, device, caller-owned)
 * for every idx[i] in [0, E) among the n device int32 indices (for example
 * the idx of moe_grouped_forward calls).  Enqueues one kernel on `stream`;
 * graph-capturable.  MOE_E_NULL / MOE_E_ALIGN for missing or misaligned
 * pointers; n == 0 is a no-op. */
moe_status moe_expert_counts(const moe_layer* layer, const int32_t* idx, int32_t n, uint32_t* counts,
                             void* stream);

/* Replace the layer's hot region by copies of the n experts ids[0, n) (host
 * int32, distinct, in [0, E); slot i holds ids[i]); n == 0 removes it.
 * Synchronises `stream` (before freeing the old region and after the
 * copies), allocates n * (bytes of one expert) + 4 E + 4 n bytes of device
 * memory owned by the layer and freed with it.  The layer's pool must hold
 * the weights that are copied.  Not concurrent with calls that use the layer;
 * graphs captured before the change keep reading the old region, so
 * recapture them.  MOE_E_RANGE for n outside [0, E], an index out of range or
 * repeated; MOE_E_NULL for ids == NULL with n > 0. */
moe_status moe_layer_set_hot_experts(moe_layer* layer, const int32_t* ids, int32_t n, void* stream);

/* ---- Host tier: experts computed by the host's cores.
 *
 * The pages compute the experts the GPU does not hold on the host's cores,
 * from 4-bit weights in host RAM with wide vector instructions, while the
 * GPU computes the rest, and add the parts at the combine (pyshine source
 * tour, Understanding the Architecture, the paragraphs on three tiers and
 * one residency table and on the CPU pool behind a doorbell). */

/* Move the n experts ids[0, n) (host int32, distinct, in [0, E), none in the
 * hot region) to the host tier; n == 0 removes it.  Their weights are copied
 * from the device pool into pinned host memory; from then on the GPU kernels
 * read an all-zero expert in their place (so their part of the GPU's sum is
 * exactly 0) and a pool of n_threads host threads (0: up to 16) computes
 * them.  In each call, on a second stream: the call's indices, gates and
 * hidden states to pinned memory, a host node that runs the pool, its
 * output back to the device; the call's stream waits for it before adding it
 * to the GPU's output (graph-capturable).  Calls on such a layer take at most
 * floor(256 / k) tokens, run the few-token kernels and must not overlap one
 * another.  Synchronises `stream`.  MOE_E_RANGE for bad ids or n_threads
 * outside [0, 1024]. */
moe_status moe_layer_set_host_experts(moe_layer* layer, const int32_t* ids, int32_t n, int32_t n_threads,
                                      void* stream);

/* The host pool's arithmetic on caller host arrays, no GPU: for each token t
 * of the T hidden states x (act_dtype, [T][H]), out[t] (fp32 [H]) = the sum
 * over j < k in order of gates[t][j] * y_e(x_t), e = idx[t][j] (host int32
 * and fp32 [T][k]; an index outside [0, E) adds nothing), with y_e =
 * D_e (silu(G_e x) * (U_e x)) in binary32 from desc's expert pools, which are
 * HOST pointers here (the router fields are not read).  n_threads threads
 * (0 or 1: the calling thread alone). */
moe_status moe_cpu_experts(const moe_layer_desc* desc, const void* x, int32_t T, const int32_t* idx,
                           const float* gates, float* out, int32_t n_threads);

/* ---- Batch-1 decode through a stack of layers, one captured graph per layer.
 *
 * The pages' engine composes each token from one captured graph per layer:
 * a graph bakes in its arguments, so per-token values arrive through
 * fixed-address device buffers, and the host decides when each layer's graph
 * runs, signalled by a doorbell (pyshine source tour, paragraph on the driver
 * that composes one token).
 *
 * A decoder chains n_layers layers (bf16 activations, one hidden size H, one
 * device) through a residual stream.  Layer l reads its input slot x_l (bf16
 * [H]), runs moe_grouped_forward (T = 1, routed inside, its own workspace)
 * into idx_l (int32 [k]), gates_l (fp32 [k]) and out_l (fp32 [H]), then its
 * epilogue writes x_{l+1} = bf16(x_l + out_l) (the fp32 sum rounded to
 * nearest even) into slot l + 1 -- slot n_layers is the decoder's result --
 * and rings the layer's doorbell: a host-pinned word that receives the step
 * number (1, 2, ...) once the layer's stores are in memory. */
typedef struct moe_decoder moe_decoder;

/* Allocate the fixed buffers (device memory, zeroed; doorbells in
 * host-pinned memory) and capture one graph per layer.  Synchronises
 * `stream` first; the layers must outlive the decoder.  The current device
 * must be the layers'.  MOE_E_RANGE for n_layers outside [1, 64] or layers on
 * another device; MOE_E_DTYPE for fp32 activations; MOE_E_GEOMETRY for
 * differing hidden sizes. */
moe_status moe_decoder_create(const moe_layer* const* layers, int32_t n_layers, void* stream,
                              moe_decoder** out);

/* Synchronise the device, then free everything the decoder owns.  NULL is a
 * no-op. */
moe_status moe_decoder_destroy(moe_decoder* decoder);

/* The fixed device addresses of layer `layer` (0 <= layer <= n_layers): its
 * input slot (bf16 [H]) and its outputs out (fp32 [H]), idx (int32 [k]),
 * gates (fp32 [k]); layer n_layers has only the result slot (the others are
 * set to NULL).  Any output pointer may be NULL.  A caller writes the
 * token's hidden state into slot 0 on the stream it steps on. */
moe_status moe_decoder_buffers(const moe_decoder* decoder, int32_t layer, void** x, float** out,
                               int32_t** idx, float** gates);

/* One token on `stream`.  wait_doorbell == 0: one launch of a graph that
 * holds every layer's graph in order (the host returns at once).
 * wait_doorbell != 0: the layers' graphs one launch each, the host launching
 * layer l + 1 only after layer l's doorbell shows this step (a bounded spin:
 * MOE_E_HIP after 2 s).  Calls on one decoder must not overlap. */
moe_status moe_decoder_step(moe_decoder* decoder, void* stream, int32_t wait_doorbell);

/* The last step layer `layer` has rung (0 before the first); a host read,
 * no synchronisation. */
moe_status moe_decoder_doorbell(const moe_decoder* decoder, int32_t layer, uint64_t* step);

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
