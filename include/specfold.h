/*
 * specfold.h -- C ABI of the folded multi-branch verify layer for AMD MI355X (gfx950).
 *
 * One verify step of a block-diffusion LLM runs a parent branch and its draft children
 * (each revealing one or a few more masked positions of the same block) through a
 * transformer layer together.  Most child positions barely differ from their parent, so
 * the layer measures the per-position difference at its input, reuses the parent's
 * projections and FFN output where the difference is small, packs the positions that
 * must be recomputed from every branch into one batch, runs the heavy GEMMs once on
 * that batch, and corrects each folded position's attention with its own branch's
 * keys and values while the shared prefix cache is read once through a strided view.
 *
 * Sources (cited by page and section):
 *   "SpecFold" explainer, blog.ontle.kr/blog/358: the paragraphs on measuring
 *     ||H_child - H_parent|| / ||H_parent|| at the layer input, on reusing the parent
 *     while keeping the child's own delta, on packing the recompute positions of all
 *     branches into one bundle, on referencing the shared prefix cache without copies,
 *     and the implementation memo (gate, provenance and streaming-attention kernels,
 *     zero-copy strided view, GQA);
 *   "SpecFold uskoryaet diffuzionnye yazykovye modeli do 1,99x", iitog.ru: the abstract
 *     summary (token-level residual gating, folded attention and FFN);
 *   Spiffy explainer, lifetechia.com/?p=5403: the directed draft graph.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or retains them beyond the call.  They must be 16-byte aligned.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *     stream).  Host-side argument checks run first and fail before anything is
 *     enqueued; device faults surface at the caller's next synchronisation.
 *   - Integer results (masks, provenance, packing) are exact; floating-point results are
 *     deterministic (bit-identical between runs, no floating-point atomics).
 *   - Calls on different streams are safe when they use different output and workspace
 *     buffers.  The only global device state is the array behind
 *     specfold_layer_forward_static (its calls on one device share it) and the result slot
 *     of the SPECFOLD_DEBUG graph check (whose use is serialised on the host).
 *   - On failure a status other than SPECFOLD_OK is returned and specfold_last_error()
 *     returns a message (per host thread).  A HIP error left pending by an earlier,
 *     unrelated HIP call on the calling thread is cleared on entry, not reported.
 *   - Device-side index inputs (fold_src, masks, provenance, packed rows) are clamped
 *     before use, so malformed values give wrong results but never out-of-bounds access.
 *     With SPECFOLD_DEBUG set in the environment (to anything but "" or "0"), calls that
 *     take fold_src first check it on the device (fold_src[0] = -1, 0 <= fold_src[n] < n)
 *     and fail with SPECFOLD_ERR_INVALID_ARGUMENT naming the first offending node before
 *     any of their kernels run; that check waits for the stream, so such calls cannot be
 *     captured into a graph.
 *
 * Layouts (row-major, elements of `dtype` unless noted):
 *   hidden states H      [N, B, d]         N = num_nodes (node 0 = parent/root), B = block
 *   slot                 s = n * B + i     (node-major, position-minor), S = N * B
 *   fold_src             int32 [N]         fold source (first parent) of each node;
 *                                          fold_src[0] = -1 and 0 <= fold_src[n] < n
 *                                          (nodes are numbered topologically)
 *   w_qkv                [(n_q + 2 n_kv) dh, d]  rows: Q heads, then K heads, then V heads
 *   w_o                  [d, n_q dh]
 *   w_gate_up            [2 ffn, d]        rows: gate projection, then up projection
 *   w_down               [d, ffn]
 *   rms1, rms2           [d]               RMSNorm gains
 *   prefix K/V           element (t, kvh, c) at ptr[t * stride_tok + kvh * stride_head + c]
 */
#ifndef SPECFOLD_H
#define SPECFOLD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum specfold_status {
  SPECFOLD_OK = 0,
  SPECFOLD_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misaligned pointer      */
  SPECFOLD_ERR_UNSUPPORTED = 2,      /* valid but unsupported shape (see below)         */
  SPECFOLD_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required      */
  SPECFOLD_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed      */
} specfold_status;

typedef enum specfold_dtype {
  SPECFOLD_F32 = 0,   /* float32 storage and arithmetic                                 */
  SPECFOLD_BF16 = 1   /* bfloat16 storage; fp32 accumulation, softmax and gate          */
} specfold_dtype;

/* Shape of one verify layer.  Supported: num_nodes >= 1, 1 <= block <= 1024,
 * num_nodes * block <= 16384, hidden and ffn multiples of 128 (hidden <= 32768,
 * ffn <= 131072), head_dim 64 or 128, n_q_heads <= 256 and a multiple of n_kv_heads,
 * 0 <= prefix_len <= 2^24, rms_eps finite and >= 0, rope_theta finite and >= 0.
 * rope_theta > 0 turns on the rotary position embedding (rotate-half form, as in the
 * Llama / Qwen model families): after the QKV projection, the Q and K heads of the packed
 * row of block position i are rotated at absolute position prefix_len + i, the pair
 * (j, j + head_dim/2) by the angle (prefix_len + i) * rope_theta^(-2j/head_dim).  The
 * prefix cache must hold keys that are already rotated.  0 = no rotary embedding. */
typedef struct specfold_shape {
  int32_t num_nodes;
  int32_t block;
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn;
  int32_t prefix_len;
  float rms_eps;
  int32_t dtype;       /* specfold_dtype */
  float rope_theta;    /* rotary embedding base; 0 = none */
} specfold_shape;

/* Zero-copy strided view of the shared prefix cache (SpecFold explainer: the shared cache
 * is referenced, never copied per branch).  Strides are in elements; the head_dim
 * elements of one (token, head) are contiguous; strides must keep rows 16-byte aligned,
 * and stride_tok must stay below 64 MB per token (SPECFOLD_ERR_UNSUPPORTED otherwise). */
typedef struct specfold_kv_view {
  const void* k;
  const void* v;
  int64_t stride_tok;
  int64_t stride_head;
} specfold_kv_view;

typedef struct specfold_layer_weights {
  const void* rms1;
  const void* w_qkv;
  const void* w_o;
  const void* rms2;
  const void* w_gate_up;
  const void* w_down;
  const void* b_qkv;   /* [(n_q + 2 n_kv) dh] bias of the Q/K/V projections, or NULL */
} specfold_layer_weights;

/* Fold state of one layer (device buffers, S = num_nodes * block entries each).
 * Outputs of specfold_layer_forward, or inputs with SPECFOLD_FLAG_FOLD_STATE_IN.
 * Any pointer may be NULL: the library then keeps that array in the workspace. */
typedef struct specfold_fold_state {
  float* ratio;          /* [S]  r = ||H_n - H_src|| / ||H_src|| (+inf for the root)  */
  uint8_t* recompute;    /* [S]  1 = recompute, 0 = folded                             */
  int32_t* src_node;     /* [S]  node whose computation the slot uses                  */
  int32_t* packed_slot;  /* [S]  packed row k -> slot id (first packed_count valid)    */
  int32_t* slot_row;     /* [S]  slot -> packed row of (src_node, position)            */
  int32_t* packed_count; /* [1]  K = number of packed (recompute) rows                 */
} specfold_fold_state;

/* Skip the fold decision, provenance and packing, and read recompute, src_node,
 * packed_slot, slot_row and packed_count from `state` (all five must be non-NULL and
 * mutually consistent).  If state->ratio and fold_src are both non-NULL, the gate's
 * ratios on this call's input are still written to state->ratio (for inspection; they
 * decide nothing). */
#define SPECFOLD_FLAG_FOLD_STATE_IN 1u

/* REUSE variant of folded attention: a folded slot takes its resolved source's attention
 * output as it is, instead of attending with its own branch's block keys and values (the
 * correction of the SpecFold explainer's implementation memo).  Only the packed rows then
 * need the O projection, h[s] = H[s] + (o W_o^T)[slot_row[s]], so the output of a folded
 * slot differs from its source's by its own input delta, y[n,i] = y[src,i] + H[n,i] -
 * H[src,i] (up to rounding).  Timing both modes measures what the correction costs. */
#define SPECFOLD_FLAG_REUSE_ATTENTION 2u

/* Gate (SpecFold explainer, paragraph on measuring the relative difference at the layer
 * input; iitog.ru summary, "token-level residual gating").
 * For every child n >= 1 and position i:
 *     r = ||H[n,i] - H[p,i]||_2 / ||H[p,i]||_2,  p = fold_src[n],
 * accumulated in fp32; recompute = !(r <= tau), so tau < 0 folds nothing, tau = +inf
 * folds every finite ratio, a NaN ratio recomputes and a NaN tau folds nothing.  ||H[p,i]|| = 0 gives r = 0 when the
 * rows are equal and +inf otherwise.  Root rows always recompute (r = +inf), and so
 * does any node whose fold_src entry is not in [0, n).
 *   hidden    [N, B, d] device, dtype = shape->dtype
 *   fold_src  [N] int32 device
 *   ratio     [N, B] float device, or NULL
 *   recompute [N, B] uint8 device (required)                                          */
specfold_status specfold_gate(const specfold_shape* shape, const void* hidden,
                              const int32_t* fold_src, float tau, float* ratio,
                              uint8_t* recompute, void* stream);

/* Provenance (SpecFold explainer, implementation memo: follow fold chains so every
 * folded position points at the ancestor state that actually computed it).
 *     src_node[n,i] = n                        if slot (n,i) recomputes (or n = 0),
 *                   = src_node[fold_src[n], i] otherwise.
 *   recompute [N, B] uint8 device; fold_src [N] int32 device; src_node [N, B] int32 device */
specfold_status specfold_resolve(const specfold_shape* shape, const uint8_t* recompute,
                                 const int32_t* fold_src, int32_t* src_node, void* stream);

/* Packing (SpecFold explainer: the recompute positions of all branches are compacted
 * into one bundle so the heavy layer runs once on it).  Stable compaction of the
 * recompute slots (root slots always count) in ascending slot id:
 *     packed_slot[k] = slot id of the k-th recompute slot, k < K
 *     slot_row[n,i]  = k such that packed_slot[k] = src_node[n,i] * B + i
 *     packed_count[0] = K
 *   recompute, src_node: [N, B] device inputs; packed_slot, slot_row: [N, B] int32
 *   device outputs (packed_slot entries >= K are left unspecified); packed_count: [1]
 *   int32 device output.  src_node must come from specfold_resolve on the same mask.  */
specfold_status specfold_pack(const specfold_shape* shape, const uint8_t* recompute,
                              const int32_t* src_node, int32_t* packed_slot,
                              int32_t* slot_row, int32_t* packed_count, void* stream);

/* Bytes of device workspace specfold_layer_forward needs for `shape` (0 if the shape is
 * invalid or unsupported; see specfold_last_error). */
size_t specfold_layer_workspace_bytes(const specfold_shape* shape);

/* One folded verify layer (all steps of the SpecFold explainer's paragraphs on reuse,
 * packing and streaming attention with per-branch correction):
 *   1-3. gate, provenance and packing as above (skipped with SPECFOLD_FLAG_FOLD_STATE_IN);
 *   4.   A = RMSNorm(H[packed rows]) * rms1;  [Q|K|V] = A w_qkv^T on the K packed rows;
 *   5.   attention of every slot (n,i) and query head h (KV head h / (n_q/n_kv)):
 *        query = Q[slot_row[n,i], h]; keys/values = the prefix view followed by branch
 *        n's own block rows K/V[slot_row[n,j]], j < B; no mask; scale 1/sqrt(head_dim);
 *        the prefix is streamed once per packed row and merged with each branch's block;
 *   6.   h = H + o w_o^T for every slot;
 *   7.   F = (SiLU(A2 w_gate^T) * (A2 w_up^T)) w_down^T, A2 = RMSNorm(h[packed rows]) * rms2;
 *   8.   hidden_out[n,i] = h[n,i] + F[slot_row[n,i]].
 * bf16: Q/K/V, attention output, h, the SwiGLU product, F and hidden_out are rounded to
 * bf16; accumulation, softmax and normalisation statistics are fp32.
 *   hidden_in, hidden_out: [N, B, d] device, no aliasing.
 *   fold_src: [N] int32 device (may be NULL only with SPECFOLD_FLAG_FOLD_STATE_IN).
 *   state: fold-state buffers (outputs, or inputs with the flag); may be NULL without it.
 *   workspace: device buffer of at least specfold_layer_workspace_bytes(shape) bytes,
 *   256-byte aligned; calls that overlap in time need distinct workspaces.             */
specfold_status specfold_layer_forward(const specfold_shape* shape,
                                       const specfold_layer_weights* weights,
                                       const specfold_kv_view* prefix,
                                       const void* hidden_in, void* hidden_out,
                                       const int32_t* fold_src, float tau,
                                       specfold_fold_state* state, uint32_t flags,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Allocation-free variant of specfold_layer_forward, for callers that cannot allocate
 * device memory around the call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks, launches and results as
 * specfold_layer_forward, but the workspace is a static device array inside the library:
 * SPECFOLD_STATIC_WORKSPACE_BYTES per GPU, reserved when the library's code is loaded on
 * that GPU and held until the process ends.  The call itself allocates and frees nothing.
 *   - Shapes whose specfold_layer_workspace_bytes exceeds SPECFOLD_STATIC_WORKSPACE_BYTES
 *     are rejected with SPECFOLD_ERR_WORKSPACE before anything is enqueued (the 7B-shaped
 *     layer with 1+15 branches needs about 85 MiB).
 *   - Every call on one GPU shares that GPU's array, and it keeps the last call's
 *     contents (nothing in it needs to start at zero).  Calls that overlap in time on one
 *     GPU -- on different streams, or from different host threads without ordering --
 *     race on it; order them on one stream.
 *   - The first call on each device looks the array's device address up once
 *     (hipGetSymbolAddress); a failure there returns SPECFOLD_ERR_HIP.              */
#define SPECFOLD_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)
specfold_status specfold_layer_forward_static(const specfold_shape* shape,
                                              const specfold_layer_weights* weights,
                                              const specfold_kv_view* prefix,
                                              const void* hidden_in, void* hidden_out,
                                              const int32_t* fold_src, float tau,
                                              specfold_fold_state* state, uint32_t flags,
                                              void* stream);

/* Bytes of device workspace specfold_stack_forward needs for `shape`: one layer's
 * workspace followed by one spare [N, B, d] hidden-state buffer (0 if the shape is
 * invalid or unsupported).  The layer part has the layout that specfold_workspace_offset
 * describes, and holds the last layer's intermediates after the call. */
size_t specfold_stack_workspace_bytes(const specfold_shape* shape);

/* A stack of folded verify layers (SpecFold explainer: the residual ripple grows through
 * the layers and the fold decision is taken again at every layer, so a position folded
 * at one layer can be recomputed at a later one).  Layer l runs specfold_layer_forward's
 * steps on layer l-1's output (layer 0 on hidden_in) with its own weights, prefix view
 * and gate; the residual stream between layers is stored in shape->dtype.
 *   num_layers >= 1.
 *   weights: host array [num_layers] of device weight sets.
 *   prefix:  host array [num_layers] of views (may be NULL when prefix_len == 0).
 *   hidden_in, hidden_out: [N, B, d] device, no aliasing with each other or the workspace;
 *   hidden_out receives the last layer's output.
 *   fold_src: [N] int32 device, the same draft graph for every layer (may be NULL only
 *   with SPECFOLD_FLAG_FOLD_STATE_IN).
 *   states: NULL, or host array [num_layers] of fold-state buffer sets: outputs of each
 *   layer's gate/provenance/packing (NULL members fall back to the workspace), or with
 *   SPECFOLD_FLAG_FOLD_STATE_IN every layer's complete input state.
 *   workspace: at least specfold_stack_workspace_bytes(shape) bytes, 256-byte aligned.
 * All arguments of all layers are checked before the first launch. */
specfold_status specfold_stack_forward(const specfold_shape* shape, int32_t num_layers,
                                       const specfold_layer_weights* weights,
                                       const specfold_kv_view* prefix,
                                       const void* hidden_in, void* hidden_out,
                                       const int32_t* fold_src, float tau,
                                       specfold_fold_state* states, uint32_t flags,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Launch steps of specfold_layer_forward, for timing probes. */
typedef enum specfold_step {
  SPECFOLD_STEP_GATE = 0,          /* gate (also every slot's RMS-normalised row)     */
  SPECFOLD_STEP_RESOLVE_PACK = 1,  /* provenance + packing                            */
  SPECFOLD_STEP_RMSNORM1 = 2,      /* fused into the gate: not recorded               */
  SPECFOLD_STEP_QKV = 3,           /* packed QKV GEMM (incl. its split-K reduction)   */
  SPECFOLD_STEP_ATTN_PREFIX = 4,   /* prefix-phase attention                          */
  SPECFOLD_STEP_ATTN_BLOCK = 5,    /* block-phase attention + merge                   */
  SPECFOLD_STEP_O_PROJ = 6,        /* O projection over all slots (fp32 partials)     */
  SPECFOLD_STEP_RMSNORM2 = 7,      /* O finish: residual add + FFN RMSNorm of packed  */
  SPECFOLD_STEP_FFN_GATE_UP = 8,   /* packed gate/up GEMM with the SwiGLU product     */
  SPECFOLD_STEP_FFN_DOWN = 9,      /* packed down GEMM                                */
  SPECFOLD_STEP_COMBINE = 10       /* y = h + F[slot_row]                             */
} specfold_step;

/* A timing probe: `start` is recorded on the stream right before the first launch of
 * step `step` and `stop` right after its last launch (both are hipEvent_t created by the
 * caller).  When the FFN gate/up step is a single kernel (the column slabs, or the tiles
 * chosen on the device), its events are instead taken at that kernel's start and end
 * (hipExtLaunchKernel), which leaves out the cost of recording two events around it.
 * Nothing is recorded for a step that the call skips. */
typedef struct specfold_probe {
  int32_t step;
  void* start;
  void* stop;
} specfold_probe;

/* specfold_layer_forward with an optional timing probe (probe may be NULL). */
specfold_status specfold_layer_forward_probed(const specfold_shape* shape,
                                              const specfold_layer_weights* weights,
                                              const specfold_kv_view* prefix,
                                              const void* hidden_in, void* hidden_out,
                                              const int32_t* fold_src, float tau,
                                              specfold_fold_state* state, uint32_t flags,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream, const specfold_probe* probe);

/* Intermediates of the last specfold_layer_forward that are kept in the workspace, for
 * inspection after the stream has synchronised.  Row k of a packed tensor is packed row
 * k (k < K); slot tensors have S rows.  All are row-major in shape->dtype with the row
 * stride returned by specfold_workspace_offset (packed activations carry one extra
 * 128-byte line per row).                                                              */
typedef enum specfold_tensor {
  SPECFOLD_T_QKV = 0,    /* [S cap, (n_q + 2 n_kv) dh] packed Q|K|V rows          */
  SPECFOLD_T_ATTN = 1,   /* [S, n_q dh] attention output of every slot            */
  SPECFOLD_T_H = 2,      /* [S, d]  h = H + attention projection                  */
  SPECFOLD_T_FFN = 3     /* [S cap, d] packed FFN output rows                     */
} specfold_tensor;

/* Byte offset of tensor `which` inside the workspace (SIZE_MAX on invalid input); the row
 * stride in elements is stored to *ld_elems when ld_elems is non-NULL. */
size_t specfold_workspace_offset(const specfold_shape* shape, int32_t which, int64_t* ld_elems);

/* Bytes of device workspace specfold_lm_head_argmax needs (0 if the shape is invalid). */
size_t specfold_lm_head_workspace_bytes(const specfold_shape* shape, int32_t vocab);

/* LM head after the last folded layer, and every branch's predicted token (the verify
 * step compares the branches' predictions; SpecFold explainer, the reuse path: a folded
 * position takes its resolved source's result, here its prediction).
 *   For packed row k < K = *packed_count (slot packed_slot[k]):
 *     a_k = hidden[slot] / sqrt(mean(hidden[slot]^2) + rms_eps) * rms_final
 *     logit[k, v] = a_k . w_lm[v]                      (fp32 accumulation)
 *     row_token[k] = the first v of the largest logit;  row_logit[k] = that logit
 *                    (NaN logits never win)
 *   token[n, i] = row_token[slot_row[n, i]] for every slot.
 * The fold state (packed_slot, slot_row, packed_count) is the last layer's, as produced
 * by specfold_layer_forward / specfold_stack_forward; with every slot packed (tau < 0)
 * every slot gets its own prediction.  The logits are never stored.
 *   shape:       num_nodes, block, hidden, rms_eps, dtype are used (hidden % 128 == 0)
 *   rms_final:   [d] dtype;  w_lm: [vocab, d] dtype, row-major;  hidden: [N, B, d] dtype
 *   row_token:   int32 [N*B] capacity, first K written (-1 if no logit of the row is above
 *                -inf, e.g. all NaN; its row_logit is then -inf)
 *   row_logit:   float [N*B] capacity or NULL;  token: int32 [N, B]
 *   workspace:   specfold_lm_head_workspace_bytes(shape, vocab) bytes, 256-byte aligned
 * Errors: SPECFOLD_ERR_INVALID_ARGUMENT for NULL / misaligned pointers or vocab outside
 * [1, 2^24], SPECFOLD_ERR_UNSUPPORTED for unsupported shapes, SPECFOLD_ERR_WORKSPACE for a
 * short workspace, SPECFOLD_ERR_HIP if a launch fails. */
specfold_status specfold_lm_head_argmax(const specfold_shape* shape, int32_t vocab,
                                        const void* rms_final, const void* w_lm,
                                        const void* hidden, const int32_t* packed_slot,
                                        const int32_t* slot_row, const int32_t* packed_count,
                                        int32_t* row_token, float* row_logit, int32_t* token,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* Message of the last failed call on this host thread ("" if none). */
const char* specfold_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t specfold_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPECFOLD_H */
