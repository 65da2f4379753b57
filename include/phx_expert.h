/*
 * phx_expert.h -- C ABI of a flow-matching action-expert decision on AMD
 * Instinct MI355X (gfx950).
 *
 * One decision integrates S flow-matching Euler steps of an NL-layer
 * decoder over M action rows per request.  Every layer's action rows attend
 * to a prefix key/value cache that is written once and read by every step,
 * and to the action rows themselves.  Sources, cited by page title and
 * section:
 *   - "FlashRT-PAI: Fast Kernels Are Not Fast Pipelines for Physical AI
 *     Inference": section 2.1 (Figure 1a: the pi0.5 decision, a prefix of
 *     about 500 to 800 tokens writing its K/V, an 18-layer expert over ten
 *     action rows and ten flow steps; a deployment fixes views, context
 *     bucket, action horizon and step count), section 3.4 and Appendix A.1
 *     (static buffers, swap windows and state regions at fixed addresses; a
 *     versioned C interface with shape and plan checks; the caller owns
 *     input freshness), section 3.2 (fused producers: residual + norm,
 *     RoPE with the QKV split and cache write, GeGLU in the GEMM epilogue).
 *   - "PhyAI" paper, section 4.2 (Graph replay: the prefix K/V, the
 *     timestep table and every layer's AdaRMS modulation table are prepared
 *     before denoising and the whole step loop is replayed as one graph;
 *     Kernel fusion: one QKV GEMM, merged gate/up with GeGLU, AdaRMSNorm).
 *
 * Ownership.  The library owns every device allocation it makes and frees it
 * in phx_expert_destroy.  Pointers passed in stay owned by the caller and must
 * stay valid until the given stream has passed the call.  Calls on one handle
 * must not overlap: the handle keeps one working set.
 *
 * Errors.  Every int-returning call returns PHX_OK (0) or a negative PHX_E_*
 * code and leaves a message for phx_last_error() in the calling thread.  On
 * error the handle is unchanged.  Nothing throws across this boundary.
 */
#ifndef PHX_EXPERT_H
#define PHX_EXPERT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define PHX_API __attribute__((visibility("default")))
#else
#define PHX_API
#endif

#define PHX_ABI_VERSION 2u

/* return codes */
#define PHX_OK 0
#define PHX_E_INVALID (-1)     /* NULL pointer or a bad argument value */
#define PHX_E_VERSION (-2)     /* abi_version or struct_size does not match this library */
#define PHX_E_SHAPE (-3)       /* outside the prepared plan: prefix_len > capacity, bad request index,
                                  or a shape the library does not support */
#define PHX_E_STATE (-4)       /* a prerequisite is missing: decide before every request has a prefix */
#define PHX_E_NOMEM (-5)       /* device allocation failed */
#define PHX_E_HIP (-6)         /* a HIP runtime call failed; the message names it */

/* element types of weights and prefix K/V */
#define PHX_DTYPE_F32 0
#define PHX_DTYPE_BF16 1

/* execution flags */
#define PHX_FLAG_NO_GRAPH 1u   /* launch the multi-kernel step loop's kernels directly instead of
                                  replaying the captured graph (same kernels, same results; for diagnosis) */
#define PHX_FLAG_MULTI_KERNEL 2u  /* run the multi-kernel graph even where the persistent decision kernel
                                     applies (for comparison) */
#define PHX_FLAG_WEIGHTS_INT8 8u  /* 8-bit weight tier (W8A16, "PhyAI" section 4.2 Quantization): every layer's
                                     W_qkv, W_o, W_gu and W_down is quantised at create to int8 codes by
                                     round-to-nearest per output column (s = max|w| / 127, q =
                                     rint(w / s), ties to even, float32 arithmetic); activations stay
                                     bf16 and each projection's sum is scaled by s in fp32.  bf16
                                     weights, decoder block, batch * rows <= 160; runs on the persistent
                                     decision kernel where that kernel applies (its tile ring then
                                     carries the codes), otherwise on the multi-kernel graph (see
                                     phx_expert_weight_codes) */
#define PHX_FLAG_TIMELINE 4u   /* persistent kernel: record a per-workgroup phase timeline (see
                                  phx_expert_timeline) */
#define PHX_FLAG_PAIRED_ACT 16u  /* large-token plans (more than 160 rows, the DiT-style block, the prefill):
                                    the inputs of the MLP's two GEMMs, gate/up and down (the MLP norm's rows
                                    and the MLP activation), are carried as pairs of bf16 values,
                                    hi = bf16(a) and lo = bf16(a - hi), and each GEMM sums hi * w + lo * w
                                    against the bf16 weights, so it sees its activation to ~2^-16 instead
                                    of 2^-8 at twice the matrix-core work; the prefill pairs its QKV
                                    input too (its keys and values are its output), the other plans keep
                                    it, like the attention output, bf16.  The default of
                                    PHX_BLOCK_DIT, of PHX_BLOCK_PREFILL and of the batched plan (bf16, 65-160
                                    rows: the rollout batch): their results accumulate the most bf16
                                    rounding; opt-in for the large-token decoder plan (the video-action
                                    chunk) */
#define PHX_FLAG_BF16_ACT 32u  /* large-token plans: plain bf16 GEMM activations everywhere (faster; more
                                  rounding in the DiT-style step, the prefill and the rollout batch) */

/* block kinds */
#define PHX_BLOCK_DECODER 0  /* adaptive RMSNorm (scale, shift), RoPE, GeGLU MLP, residual adds; in- and
                                out-linears around the stack and an Euler update per step (the pi0.5
                                action expert, and the video-action chunk at width 2048) */
#define PHX_BLOCK_DIT 1      /* DiT-style adaLN-Zero block: LayerNorm without affine modulated by
                                (1 + scale) and shift, gated attention and GELU-MLP residual branches,
                                no rotary positions; one pass over the tokens, no in/out linears and no
                                Euler update (state_dim = width, steps = 1, prefix_capacity = 0) */
#define PHX_BLOCK_PREFILL 2  /* prefix prefill: the decoder stack that reads the prefix tokens and writes
                                the key/value cache an action expert attends to ("FlashRT-PAI", section
                                2.1, Figure 1a); RMSNorm with a learned gain (1 + g), RoPE at positions
                                0.., causal attention, GeGLU MLP, residual adds; no in/out linears
                                (state_dim = width, steps = 1, prefix_capacity = 0, mask
                                PHX_MASK_CAUSAL, rows = the most prefix tokens one call takes) */

/* attention masks */
#define PHX_MASK_FULL 0      /* every row sees every prefix key and every row of its own chunk */
#define PHX_MASK_CAUSAL 1    /* token i sees tokens 0..i (the prefix prefill, and only it) */

/* A HIP stream (hipStream_t is a pointer to this incomplete type). NULL means
   the default stream. */
typedef struct ihipStream_t* phx_stream_t;

/*
 * Deployment shape, fixed for the life of a handle.  Notation of the pages'
 * pi0.5 shape in brackets.
 */
typedef struct phx_expert_config {
  uint32_t abi_version;      /* PHX_ABI_VERSION */
  uint32_t struct_size;      /* sizeof(phx_expert_config) */
  int32_t layers;            /* NL decoder layers [18] */
  int32_t width;             /* D residual width [1024]; multiple of 128 */
  int32_t n_heads;           /* H query heads [8] */
  int32_t head_dim;          /* Dh [256]; 64, 128 or 256; n_heads*head_dim a multiple of 128 */
  int32_t n_kv_heads;        /* KVH key/value heads [1: multi-query]; divides H */
  int32_t mlp_hidden;        /* F GeGLU hidden width [4096]; multiple of 128 */
  int32_t state_dim;         /* A action dimension [32]; multiple of 32 */
  int32_t rows;              /* M action rows per request [10] (tokens of the chunk for the large-token
                                workloads); B*M <= 160 with n_heads/n_kv_heads*rows <= 128, or B = 1 and
                                161 <= M <= 16384 (large-token plan: bf16, head_dim 128, width,
                                mlp_hidden and state_dim multiples of 128) */
  int32_t batch;             /* B requests per decision */
  int32_t prefix_capacity;   /* C context bucket: most prefix rows a request may load [768]; <= 65536 */
  int32_t steps;             /* S Euler steps [10] */
  int32_t time_emb_dim;      /* E sinusoidal time-embedding width [1024]; even */
  float tau0;                /* flow time of the first step [1.0] */
  float dt;                  /* Euler step [-0.1]: tau_k = tau0 + k*dt, x += dt*v */
  float rms_eps;             /* [1e-6], inside the square root */
  float rope_base;           /* [10000] */
  int32_t weight_dtype;      /* PHX_DTYPE_F32 or PHX_DTYPE_BF16 */
  int32_t kv_dtype;          /* must equal weight_dtype */
  uint32_t flags;            /* PHX_FLAG_* */
  int32_t block_kind;        /* PHX_BLOCK_DECODER, PHX_BLOCK_DIT or PHX_BLOCK_PREFILL */
  int32_t mask_kind;         /* PHX_MASK_FULL, or PHX_MASK_CAUSAL for PHX_BLOCK_PREFILL */
} phx_expert_config;

typedef struct phx_expert phx_expert;

/*
 * Checks a configuration without touching the GPU (pure host code).
 * Returns PHX_OK, PHX_E_INVALID (NULL), PHX_E_VERSION or PHX_E_SHAPE.
 */
PHX_API int phx_expert_validate_config(const phx_expert_config* cfg);

/*
 * Size in bytes of the weight blob phx_expert_create expects for cfg.
 * The blob is one contiguous array of weight_dtype elements; every matrix is
 * [in][out] row-major (a projection is y = x . W):
 *   W_in   [A][D]
 *   for each layer: W_qkv [D][(H+2*KVH)*Dh]  (q heads, then k heads, then v heads)
 *                   W_o   [H*Dh][D]
 *                   W_gu  [D][2F]            (gate g = first F columns, up u = last F)
 *                   W_down[F][D]
 *   W_out  [D][A]
 *   W_mod  [2*NL+1][E][2D]  (norm 2l precedes attention in layer l, 2l+1 the MLP,
 *                            2*NL the velocity head; first D outputs scale, last D shift)
 * For PHX_BLOCK_DIT:
 *   for each block: W_qkv [D][3*H*Dh] (q, k, v heads), W_o [H*Dh][D], W_up [D][F], W_down [F][D]
 *   W_mod  [NL][E][6D]      (block b: shift, scale, gate of the attention branch, then shift,
 *                            scale, gate of the MLP branch, D outputs each)
 * For PHX_BLOCK_PREFILL:
 *   for each layer: W_qkv, W_o, W_gu, W_down as for the decoder
 *   G      [2*NL][D]        (RMSNorm gains: row 2l before attention, 2l+1 before the MLP; the norm
 *                            is y / rms(y) * (1 + g))
 * There are no biases.
 */
PHX_API int phx_expert_weights_bytes(const phx_expert_config* cfg, size_t* bytes);

/*
 * Builds a handle: allocates its device arenas, copies and re-tiles the
 * weights into the layout its kernels stream, builds the step-conditioning
 * table (sinusoidal embedding of every tau_k and all 2*NL+1 modulation
 * projections, kept for the life of the handle), and captures the step loop
 * as one HIP graph.  Defined by: "FlashRT-PAI" section 2.2 and Appendix A.1
 * (a deployment fixes views, context bucket, action horizon and step count;
 * a versioned interface checks shapes and plans before anything runs) and
 * section 3.4 / Table 9 (static buffers and state regions live at fixed
 * addresses for the life of the deployment); "PhyAI" paper section 4.2,
 * Graph replay (the timestep table and every layer's AdaRMS modulation are
 * prepared once, before any denoising, and the step loop is captured once).
 *   weights: host or device pointer to weights_bytes bytes in the layout
 *            above; the caller may free it once the call returns.
 *   stream:  stream the set-up work is ordered on; the call returns after it
 *            has finished.
 * Returns PHX_OK, PHX_E_INVALID, PHX_E_VERSION, PHX_E_SHAPE, PHX_E_NOMEM or
 * PHX_E_HIP.  *out is set only on success.
 */
PHX_API int phx_expert_create(const phx_expert_config* cfg, const void* weights, size_t weights_bytes,
                      phx_stream_t stream, phx_expert** out);

/*
 * Loads (replaces) the prefix context of one request: the prefix keys and
 * values every layer attends to, already rotary-encoded as the prefix model
 * wrote them.  Defined by: "FlashRT-PAI" section 2.1 / Figure 1a (the prefix
 * writes its K/V once per observation and every flow step of the expert
 * reads it) and section 3.4 (a new observation invalidates the context; the
 * caller owns the freshness of what it loads).
 *   request:    0 <= request < batch.
 *   k, v:       device pointers, [layers][prefix_len][n_kv_heads*head_dim] of
 *               kv_dtype; copied into the handle's state region (V is stored
 *               transposed).  May be NULL when prefix_len == 0.
 *   prefix_len: 0 <= prefix_len <= prefix_capacity; the request's action rows
 *               sit at positions prefix_len .. prefix_len+rows-1.
 * Asynchronous on stream.  Returns PHX_OK, PHX_E_INVALID, PHX_E_SHAPE or
 * PHX_E_HIP.
 */
PHX_API int phx_expert_load_prefix_kv(phx_expert* h, int32_t request, const void* k, const void* v,
                              int32_t prefix_len, phx_stream_t stream);

/*
 * One decision: x = noise; S Euler steps of the expert; actions = x.  For
 * PHX_BLOCK_DIT, one pass of the block stack over the tokens: noise holds the
 * token rows x, actions receives the residual stream after the last block.
 * Defined by: "FlashRT-PAI" section 2.1 / Figure 1a (ten flow-matching Euler
 * steps of the 18-layer expert over ten action rows, x += dt * v) and
 * section 3.3 (the whole decision replays without host work between
 * sublayers); "PhyAI" paper section 4.2, Graph replay (one captured graph of
 * the denoising loop per decision).
 *   noise, actions: device pointers to float32 [batch][rows][state_dim]
 *                   (they may be the same buffer).
 * Stream-ordered and asynchronous: copy in, graph replay, copy out.  The
 * caller synchronizes.  Returns PHX_OK, PHX_E_INVALID, PHX_E_STATE (a
 * request has no loaded prefix) or PHX_E_HIP.
 * PHX_OK means the decision was enqueued, not that it completed: on the
 * persistent decision kernel (kernels_per_decision == 2) a decision whose
 * workgroups could not all make progress gives up after a bounded wait and
 * writes NaN actions.  After synchronizing, phx_expert_status reports it.
 */
PHX_API int phx_expert_decide(phx_expert* h, const float* noise, float* actions, phx_stream_t stream);

/*
 * The decision of phx_expert_decide for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arithmetic, same result bit for bit; the decision
 * kernel's exchange and control words (9,666,816 bytes) live in a static
 * device array that the library holds once per device until the process
 * ends, instead of the handle's arena.  The call allocates nothing and makes
 * no runtime call that allocates: two stream-ordered copies (noise in,
 * actions out) and three kernel launches (a prepare kernel, the decision
 * kernel, its tag advance).  The array's address is looked up and the array
 * cleared when the first handle on the device is created.  When the previous
 * decision on the array had another shape (rows, prefix chunks, steps,
 * layers), the prepare kernel clears it first (a few microseconds).
 *   noise, actions: as phx_expert_decide (device memory, or pinned host
 *                   memory under capture).
 * Every call on one device shares that device's array and its decision
 * counter, and the array keeps what the last call left; calls that overlap
 * on one device (different streams without ordering between them) race and
 * give up after the bounded wait.  Only a handle on the persistent decision
 * kernel (kernels_per_decision == 2) fits the array: any other handle gets
 * PHX_E_SHAPE with a message naming the limit.  Returns PHX_OK,
 * PHX_E_INVALID, PHX_E_SHAPE, PHX_E_STATE (no prefix loaded) or PHX_E_HIP
 * (the array could not be set up on this device).  phx_expert_status
 * reports the outcome as for phx_expert_decide.
 */
PHX_API int phx_expert_decide_noalloc(phx_expert* h, const float* noise, float* actions, phx_stream_t stream);

/*
 * Prefix prefill ("FlashRT-PAI", section 2.1, Figure 1a: the language model
 * reads the prefix tokens and writes the key/value cache the action expert
 * attends to; the cache is written once per observation).  Runs the
 * PHX_BLOCK_PREFILL stack over the first prefix_len token rows of x and
 * writes every layer's keys (after RoPE, positions 0..prefix_len-1) and
 * values, in the layout phx_expert_load_prefix_kv takes.
 *   x:          device or host float32 [prefix_len][width], the token rows.
 *   prefix_len: 0 <= prefix_len <= rows (0 does nothing).  Under the causal
 *               mask the result for the first prefix_len tokens does not
 *               depend on the bucket size rows.
 *   k, v:       device pointers to [layers][prefix_len][n_kv_heads*head_dim]
 *               of kv_dtype (bf16), owned by the caller; written on stream.
 * Stream-ordered and asynchronous.  Returns PHX_OK, PHX_E_INVALID (NULL
 * argument, host k or v, or a handle of another block kind), PHX_E_SHAPE or
 * PHX_E_HIP.  phx_expert_decide and phx_expert_load_prefix_kv reject a
 * prefill handle with PHX_E_INVALID.
 */
PHX_API int phx_expert_prefill(phx_expert* h, const float* x, int32_t prefix_len, void* k, void* v,
                               phx_stream_t stream);

/* Frees every device allocation of the handle. NULL-safe. Synchronizes the
   handle's internal stream first.  Defined by: "FlashRT-PAI" Appendix A.1
   (the engine owns the deployment's buffers from set-up to teardown; the
   caller's pointers are never freed by it). */
PHX_API void phx_expert_destroy(phx_expert* h);

/* Message of the last failing call in this thread ("" if none). */
PHX_API const char* phx_last_error(void);

/*
 * History update of a chunk policy ("FlashRT-PAI", section 2.1, Figure 1b: the
 * cache over earlier chunks persists from one decision to the next and grows
 * up to a fixed window).  Commits chunk (device or host float32
 * [rows][state_dim], normally the actions of the last decision) into request
 * 0's cache: one pass of the layer stack over it at the end flow time tau0 +
 * steps * dt writes every layer's keys and values of the chunk rows after the
 * L cached rows, and L grows by rows.  When L would pass prefix_capacity (the
 * window) the oldest rows are dropped; kept rows keep their positions, and the
 * next chunk's rows sit after them.  Stream-ordered.  Only for the
 * large-token decoder plan (one request of more than 160 rows): PHX_E_SHAPE
 * otherwise, or when rows > prefix_capacity; PHX_E_STATE before a prefix is
 * loaded.  phx_expert_load_prefix_kv starts a new history at position 0.
 */
PHX_API int phx_expert_commit_chunk(phx_expert* h, const float* chunk, phx_stream_t stream);

/*
 * The 8-bit tier's codes of one matrix, for checking: layer 0 <= layer <
 * layers, matrix 0 = W_qkv, 1 = W_o, 2 = W_gu, 3 = W_down.  codes: device
 * int8 [K][N] in the blob's row-major order; scales: device float [N].
 * Stream-ordered.  Returns PHX_OK, PHX_E_INVALID, PHX_E_SHAPE (bad layer or
 * matrix), PHX_E_STATE (the handle was not created with
 * PHX_FLAG_WEIGHTS_INT8) or PHX_E_HIP.
 */
PHX_API int phx_expert_weight_codes(const phx_expert* h, int32_t layer, int32_t matrix, int8_t* codes, float* scales,
                                    phx_stream_t stream);

/* Number of kernel launches one decision replays (graph nodes). */
PHX_API int phx_expert_kernels_per_decision(const phx_expert* h, int* count);

/*
 * Diagnostics: the kernel launches of one decision, in replay order, so a
 * caller can time or profile them one at a time.
 */
#define PHX_NODE_IN_PROJ 1           /* h = x . W_in */
#define PHX_NODE_NORM_QKV_ROPE 2     /* adaptive RMSNorm, one QKV projection, RoPE on q and k */
#define PHX_NODE_ATTENTION 3         /* split-KV multi-query attention over prefix + action rows */
#define PHX_NODE_ATTN_COMBINE 4      /* fixed-order merge of the key splits */
#define PHX_NODE_OUT_PROJ_RESID 5    /* h += o . W_o */
#define PHX_NODE_NORM_GATEUP_GEGLU 6 /* adaptive RMSNorm, merged gate/up projection, GeGLU */
#define PHX_NODE_DOWN_PROJ_RESID 7   /* h += a . W_down */
#define PHX_NODE_NORM_OUT_EULER 8    /* final adaptive RMSNorm, velocity projection, x += dt * v */
#define PHX_NODE_DECISION 9          /* the persistent kernel that runs a whole decision (launching it
                                        diagnostically also advances the decision counter) */
#define PHX_NODE_TAG_ADVANCE 10      /* advances the persistent kernel's decision counter (its exchange
                                        generations); it belongs to the decision it follows, so
                                        phx_expert_launch_node does nothing for it */
/* launches of the large-token plan (more than 160 rows, or the DiT-style block) */
#define PHX_NODE_ROW_NORM 11         /* adaptive RMSNorm or LayerNorm of the residual rows into bf16 rows */
#define PHX_NODE_QKV 12              /* QKV projection of the normalised rows (RoPE on q and k in the decoder) */
#define PHX_NODE_GATEUP 13           /* gate/up projection with GeGLU, or up projection with GELU */
#define PHX_NODE_OUT_EULER 14        /* velocity projection and x += dt * v */
#define PHX_NODE_STATE_CVT 15        /* state x to bf16 rows for the input projection */

typedef struct phx_node_info {
  int32_t kind;    /* PHX_NODE_* */
  int32_t step;    /* Euler step index */
  int32_t layer;   /* decoder layer, -1 outside the layer stack */
  int32_t reserved;
  uint64_t bytes;  /* algorithmic HBM bytes of one launch: the weights it streams (plus the
                      modulation rows of a norm), or the valid prefix and action K/V rows */
  char name[32];
} phx_node_info;

/* Describes launch `node` (0 <= node < kernels_per_decision).  Returns PHX_OK,
   PHX_E_INVALID or PHX_E_SHAPE. */
PHX_API int phx_expert_node_info(const phx_expert* h, int32_t node, phx_node_info* info);

/*
 * Launches kernel `node` of the step loop once on stream, with the arguments
 * it has in the captured graph.  It reads the handle's weights and prefix
 * state and overwrites its working buffers (the state x, residual stream,
 * queries, attention partials, action-row cache slots), so the next decision
 * is unaffected: decide starts by copying in the noise.  Returns PHX_OK,
 * PHX_E_INVALID, PHX_E_SHAPE, PHX_E_STATE or PHX_E_HIP.
 */
PHX_API int phx_expert_launch_node(phx_expert* h, int32_t node, phx_stream_t stream);

/*
 * Status of the last decision of the persistent decision kernel
 * (synchronous; call after the stream has passed the decision).  0 means it
 * completed; 1 means a workgroup waited longer than its limit (0.5 s) for
 * data another workgroup should have produced, the decision gave up, and its
 * actions were filled with NaN.  That happens only when the GPU cannot hold
 * all 256 workgroups of the decision kernel at once (another process holds
 * compute units); phx_expert_create checks that one workgroup fits on every
 * compute unit.  Always 0 for the graph paths.
 * Returns PHX_OK, PHX_E_INVALID or PHX_E_HIP.
 */
PHX_API int phx_expert_status(const phx_expert* h, uint32_t* status);

/*
 * Phase timeline of the last decision of a handle created with
 * PHX_FLAG_TIMELINE (synchronous).  The persistent kernel is one launch, so
 * a profiler sees one kernel; this records, per workgroup, the 100 MHz
 * real-time counter (low 32 bits) when its compute waves finished each phase:
 * out[wg * E + e] with E = 3 + steps * (2 + 8 * layers) events: e = 0 start;
 * for step k, base b = 1 + k * (2 + 8 * layers): b input projection, then
 * b + 1 + 8 l + {0 qkv, 1 attention, 2 merge, 3 out projection, 4 its
 * all-reduce across XCDs, 5 gate/up, 6 down, 7 its all-reduce} for layer l,
 * then b + 1 + 8 * layers velocity head; E - 2 compute end, E - 1 weight
 * streaming end.  256 workgroups (workgroup b is rank b / 8 on XCD
 * (b + o) mod 8, the offset o fixed per launch).
 * If out is NULL or capacity is too small, *count receives the size needed
 * and PHX_E_SHAPE is returned.  Returns PHX_OK, PHX_E_INVALID, PHX_E_STATE
 * (no timeline), PHX_E_SHAPE or PHX_E_HIP.
 */
PHX_API int phx_expert_timeline(const phx_expert* h, uint32_t* out, size_t capacity, size_t* count);

/*
 * Execution-state capsules ("FlashRT-PAI", section 3.4 and Table 6): snapshot,
 * restore and fork of a handle's declared state regions, the ones
 * phx_expert_load_prefix_kv writes and every decision reads -- the stored
 * prefix K/V (in the handle's own layout), the prefix lengths and the decoder
 * position table -- by device-to-device copies into one caller-owned device
 * buffer.  The buffer starts with a header: a magic word, a plan fingerprint
 * (a hash of the configuration, the execution path and the region sizes),
 * the region list (names, offsets, lengths) and each request's prefix length
 * and loaded flag.  Weights and step tables stay resident and are not part of
 * a capsule.  Capsules are process-local and plan-specific: restore accepts
 * only a capsule whose fingerprint matches the handle's, i.e. one saved by a
 * handle created with the same configuration (fork = save on one handle,
 * restore on another).  A decision after restore reproduces, bit for bit, the
 * decision the saving handle would have made.  The DiT-style block keeps no
 * state between decisions: its capsule is the header alone.
 */
typedef struct phx_capsule_region {
  char name[24];
  uint64_t offset;  /* bytes from the start of the capsule */
  uint64_t bytes;
} phx_capsule_region;

/* Size in bytes of this handle's capsule. */
PHX_API int phx_expert_capsule_bytes(const phx_expert* h, size_t* bytes);
/* The capsule's regions; with out == NULL only *count is set.  PHX_E_SHAPE if
   capacity is too small. */
PHX_API int phx_expert_capsule_regions(const phx_expert* h, phx_capsule_region* out, int32_t capacity,
                                       int32_t* count);
/* Snapshot: stream-ordered copies of the state regions into capsule (device
   memory of at least phx_expert_capsule_bytes bytes).  Asynchronous; the
   caller keeps capsule alive until stream has passed the call. */
PHX_API int phx_expert_capsule_save(phx_expert* h, void* capsule, size_t bytes, phx_stream_t stream);
/* Restore (or fork into this handle): waits for stream to read the header,
   checks the magic word and the plan fingerprint (PHX_E_SHAPE on a mismatch,
   PHX_E_INVALID for a buffer that is not a capsule), then copies the regions
   back in stream order and restores each request's prefix length and loaded
   flag.  On error the handle is unchanged. */
PHX_API int phx_expert_capsule_restore(phx_expert* h, const void* capsule, size_t bytes, phx_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif
