/*
 * moe.h — C ABI of the MI355X (gfx950) DeepSeekMoE layer forward.
 *
 * The layer (definitions from "DeepSeekMoE 深度解读报告", sections 2.2, 2.3
 * and 3.1, and the Expert module of the youleyou page "DeepSeek MoE模型优化
 * 与未来演进及字节超稀疏内存技术"):
 *
 *   s[t,e]  = softmax_e( x[t]·C[e] + b[e] )               over E routed experts
 *   top-K   = the K largest s[t,e] (ties: lower e first), gate = s, no renorm
 *             (two other gates are selectable: see the flags below)
 *   FFN_W   = W2 · ( silu(W1·x) ⊙ (W3·x) ),  silu(z) = z / (1 + e^-z)
 *   out[t]  = x[t] + Σ_{s<Ks} FFN_shared_s(x[t]) + Σ_k gate[t,k]·FFN_{idx[t,k]}(x[t])
 *
 * E = N·m fine-grained routed experts of inter-dim I (an FFN of inter I·m
 * split m ways along its intermediate dimension, section 2.2); Ks shared
 * experts of inter-dim Is that bypass the router (section 2.3).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates or frees device memory, never synchronises and
 *     keeps no state between calls (apart from the optional benchmark
 *     recorder below); work is enqueued on `stream` (a
 *     hipStream_t passed as void*, NULL = the null stream) and faults surface
 *     at the caller's next synchronisation.  Calls on different streams are
 *     independent when each uses its own workspace.
 *   - bf16 tensors are bfloat16 bit patterns, row-major and contiguous, in
 *     the nn.Linear [out_features, in_features] layout; their pointers must
 *     be 16-byte aligned.  float / int32 pointers must be 4-byte aligned; the
 *     workspace 256-byte aligned.
 *   - Every argument is validated before anything is enqueued.  On any error
 *     nothing is launched and no output is written.  No C++ exception crosses
 *     the ABI.
 *   - Shape limits: 1 <= T <= 2^24; d a multiple of 64 in [64, 65536];
 *     1 <= E <= 256; 0 <= K <= E; I a multiple of 64 in [64, 65536];
 *     0 <= Ks <= 16; Is a multiple of 64 in [64, 65536] when Ks > 0 (ignored
 *     when Ks == 0); T*(K+Ks) <= 2^30; and each of x, the routed and shared
 *     parts of H, and one expert's weight matrix below 2^31 bytes (the GEMMs
 *     address them with 32-bit offsets).  gfx950 devices only.
 *   - NaN / Inf inputs are outside the contract.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer shape.  T tokens of width d; E routed experts of inter-dim I, K of
 * them active per token; Ks shared experts of inter-dim Is. */
typedef struct {
    int32_t T, d, E, I, K, Ks, Is;
    uint32_t flags;
} moe_shape_t;

/* flags (all other bits must be 0):
 *
 * MOE_FLAG_NO_RESIDUAL: out excludes the residual x (out = shared + routed).
 * Used to check the expert contributions on their own.
 *
 * MOE_FLAG_RENORM: the K gates of a token are divided by their sum (taken in
 * selection order), so they sum to one.  With the softmax gate this equals a
 * softmax over the K selected logits, the routing code of the eliteato
 * DeepSeek-V2 explainer (section 3.1).
 *
 * MOE_FLAG_SIGMOID: affinity a_e = x.C[e]; score s_e = 1 / (1 + e^-a_e); the
 * K experts with the largest s_e + expert_bias[e] are selected (ties: lower
 * e first) and gate = s_e: the bias steers the selection only (the
 * auxiliary-loss-free routing remark of the youleyou page, and the sigmoid
 * gate of the V3 line in "DeepSeekMoE 深度解读报告", closing notes).  Usually
 * combined with MOE_FLAG_RENORM.  Without this flag the bias is added to the
 * logits before the softmax and so enters both selection and gates. */
#define MOE_FLAG_NO_RESIDUAL 1u
#define MOE_FLAG_RENORM 2u
#define MOE_FLAG_SIGMOID 4u
/* MOE_FLAG_ACT8 (moe_forward_fp8 only; other entry points reject it with
 * MOE_ERR_SHAPE): the routed experts' products take 8-bit activations.
 * Each token row x gets the scale 2^e, e the smallest integer with
 * max_j |x_j| <= 448 * 2^e (448: E4M3's largest finite value; e = 0 for an
 * all-zero row), and the codes are the nearest E4M3 values of x * 2^-e,
 * ties to the even code; W1 x and W3 x are then computed from those codes
 * and the 8-bit weights on the FP8 matrix cores.  Each routed row of
 * h = silu(W1 x) * W3 x, held in bf16, is quantised by the same rule before
 * W2.  The shared experts keep bf16 activations.  (The pages only advise
 * low-bit routed experts with per-channel or per-group scales, eliteato
 * DeepSeek-V2 explainer section 5.5; power-of-two per-row scales keep every
 * quantised value and every product exact.) */
#define MOE_FLAG_ACT8 8u

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                  */
    MOE_ERR_SHAPE = 2,       /* shape outside the limits above, or bad flags */
    MOE_ERR_ALIGN = 3,       /* a pointer is not aligned as required        */
    MOE_ERR_WORKSPACE = 4,   /* workspace smaller than moe_workspace_size() */
    MOE_ERR_NO_DEVICE = 5,   /* no HIP device is visible / current          */
    MOE_ERR_DEVICE_ARCH = 6, /* the current device is not gfx950            */
    MOE_ERR_HIP = 7,         /* a HIP launch failed                         */
    MOE_ERR_SCRATCH = 8      /* moe_forward_noalloc: the shape needs more
                                scratch than its static buffer holds        */
} moe_status_t;

/* Bytes of device workspace moe_forward / moe_forward_fp8 need for this
 * shape
 * (routing scratch, the token permutation, tile lists, and the bf16
 * intermediates H [T·K·I + T·Ks·Is] and Y [T·(K+Ks), d]).  Pure host
 * arithmetic, no HIP call.  Returns 0 when the shape is invalid. */
size_t moe_workspace_size(const moe_shape_t* shape);

/* One entry of a grouped-GEMM work list: rows m0 .. m0 + nrows - 1 of group
 * `group` (0..E-1 routed expert, E..E+Ks-1 shared expert) by output columns
 * n0 .. n0 + tile_cols - 1 (of I or Is for gate/up, of d for down). */
typedef struct {
    int32_t group, m0, n0, nrows;
} moe_tile_t;

/* Where moe_forward and moe_forward_fp8 leave the token permutation (the
 * step that gathers each expert's tokens after the top-K: eliteato.com
 * DeepSeek-V2 explainer, section 3.1) inside their workspace: byte offsets
 * from its start, valid after the call has completed on its stream.
 *   idx, gate   [T, K] int32 / float32 routing; used (and so filled) only
 *               when the call's topk_idx / topk_gate are NULL
 *   goff        [E + Ks + 1] int32: first permuted row of each group,
 *               goff[E + Ks] = rows; routed groups hold their tokens in
 *               increasing token order, shared group s holds every token,
 *               row goff[E + s] + t being token t
 *   tok_of      [rows] int32: the token of each permuted row
 *   slot_of     [T, K] int32: the permuted row of (token t, choice k)
 *   tiles_gate_up, tiles_down  [max_tiles_*] moe_tile_t work lists, their
 *               first ntiles[0] / ntiles[1] entries filled, in an order of
 *               the kernels' choosing
 *   ntiles      [2] int32
 * Pure host arithmetic.  MOE_ERR_NULL if layout is NULL, MOE_ERR_SHAPE if
 * the shape is invalid.  For inspection (tests, debugging); the layout may
 * change between library versions. */
typedef struct {
    size_t idx, gate, goff, tok_of, slot_of, tiles_gate_up, tiles_down, ntiles;
    size_t act8_codes, act8_exps;   /* MOE_FLAG_ACT8 and K > 0: uint8 [T, d] codes and int32 [T]
                                       scale exponents of the 8-bit activations (else 0) */
    size_t h;                       /* bf16 [T K, I]: h of the routed rows, in permuted row order */
    size_t act8_h_codes, act8_h_exps;  /* MOE_FLAG_ACT8, K > 0 and the FP8 down tiles in use
                                       (tile_rows_down 256, I a multiple of 128): uint8 [T K, I]
                                       codes and int32 [T K] exponents of those rows (else 0;
                                       then h itself is replaced by its dequantised value) */
    int32_t rows;                                   /* T K + T Ks */
    int32_t max_tiles_gate_up, max_tiles_down;
    int32_t tile_rows_gate_up, tile_cols_gate_up;   /* gate/up tiles read tile_cols rows of W1 and of W3 */
    int32_t tile_rows_down, tile_cols_down;
} moe_layout_t;

moe_status_t moe_workspace_layout(const moe_shape_t* shape, moe_layout_t* layout);

/* Bytes of device workspace moe_route needs for this shape: the routing
 * scratch alone (no permutation, tile lists or H / Y).  Pure host
 * arithmetic.  Returns 0 when the shape is invalid or K == 0. */
size_t moe_route_workspace_size(const moe_shape_t* shape);

/* Full layer forward (the definition at the top of this file).
 *
 *   x          bf16 [T, d]        tokens
 *   centroids  bf16 [E, d]        expert centroids (may be NULL iff K == 0)
 *   expert_bias fp32 [E] or NULL  fixed per-expert logit bias added before
 *                                 the softmax (affects selection and gates)
 *   w1, w3     bf16 [E, I, d]     routed gate / up projections (NULL iff K == 0)
 *   w2         bf16 [E, d, I]     routed down projections      (NULL iff K == 0)
 *   ws1, ws3   bf16 [Ks, Is, d]   shared experts               (NULL iff Ks == 0)
 *   ws2        bf16 [Ks, d, Is]
 *   out        bf16 [T, d]        result, rounded once from fp32 (nearest-even)
 *   topk_idx   int32 [T, K] or NULL  selected experts, descending score
 *   topk_gate  fp32  [T, K] or NULL  their softmax scores
 *   workspace / workspace_bytes   device scratch of moe_workspace_size() bytes
 *
 * Arithmetic: affinities by bf16 MFMA with fp32 accumulation, softmax (or
 * sigmoid), top-K and renormalisation in fp32; expert GEMMs bf16 x bf16 -> fp32, SwiGLU in fp32, the
 * intermediates H and Y stored as bf16; the combine accumulates in fp32.
 * Results are bit-identical from run to run (no atomics decide any order). */
moe_status_t moe_forward(const moe_shape_t* shape, const void* x, const void* centroids,
                         const float* expert_bias, const void* w1, const void* w3,
                         const void* w2, const void* ws1, const void* ws3, const void* ws2,
                         void* out, int32_t* topk_idx, float* topk_gate, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Full layer forward with 8-bit routed-expert weights (for decode, where
 * reading the weights bounds the layer: it halves the bytes every routed
 * weight costs).
 *
 * Routed experts are stored as OCP FP8 E4M3 codes (sign bit 7, exponent
 * bits 6-3 with bias 7, mantissa bits 2-0; codes 0x7F / 0xFF are NaN and
 * outside the contract) with one fp32 scale per output row — per-channel
 * quantisation of the routed experts, shared experts kept at 16 bits, as the
 * eliteato DeepSeek-V2 explainer advises (section 5.5):
 *
 *   W1[e][i][j] = e4m3(w1q[e][i][j]) * w1_scale[e][i]     w1q, w3q uint8 [E, I, d]
 *   W3[e][i][j] = e4m3(w3q[e][i][j]) * w3_scale[e][i]     w1_scale, w3_scale fp32 [E, I]
 *   W2[e][o][i] = e4m3(w2q[e][o][i]) * w2_scale[e][o]     w2q uint8 [E, d, I], w2_scale fp32 [E, d]
 *
 * Everything else — shape, flags, x, centroids, bias, the bf16 shared
 * experts ws1/ws3/ws2, out, routing outputs, workspace (the same
 * moe_workspace_size()), stream, validation and errors — is as for
 * moe_forward.  w1q/w3q/w2q must be 16-byte aligned, the scales 4-byte
 * aligned; all six may be NULL iff K == 0.
 *
 * Arithmetic: each code is widened exactly to bf16, the expert GEMMs run in
 * bf16 with fp32 accumulation, and the row scale multiplies the fp32
 * accumulator of its output column before SwiGLU (gate/up) or before the
 * bf16 rounding of Y (down).  The tile follows the batch as for
 * moe_forward: few rows per expert take the 32-row tile, which streams each
 * weight once per 32 rows; many rows take the 256 x 256 tile, which widens
 * the codes from LDS, so the 8-bit layer costs what the bf16 one does there.
 * Shared experts always take the bf16 tiles. */
moe_status_t moe_forward_fp8(const moe_shape_t* shape, const void* x, const void* centroids,
                             const float* expert_bias, const void* w1q, const float* w1_scale,
                             const void* w3q, const float* w3_scale, const void* w2q,
                             const float* w2_scale, const void* ws1, const void* ws3,
                             const void* ws2, void* out, int32_t* topk_idx, float* topk_gate,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Full layer forward that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory at call time: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Arguments, arithmetic, validation and results are those of moe_forward
 * (bit-identical outputs); the workspace is instead a static device array of
 * moe_noalloc_scratch_bytes() bytes (64 MiB) that the library's code object
 * carries: each GPU it runs on holds one copy until the process ends.  Shapes
 * whose moe_workspace_size() exceeds it are rejected with MOE_ERR_SCRATCH
 * before anything is launched (the V3-shape 256-token decode batch, 45 MB,
 * fits; prefill-sized batches do not).  The first call on a device looks up
 * that device's copy (hipGetSymbolAddress); no call allocates or frees
 * memory.  Every call on one GPU shares its one copy: calls that overlap in
 * time on one GPU (on different streams, or from several host threads) race
 * on it and give undefined results — serialise them.  Nothing in the
 * scratch needs to start zeroed: every piece of it is written before it is
 * read within a call. */
moe_status_t moe_forward_noalloc(const moe_shape_t* shape, const void* x, const void* centroids,
                                 const float* expert_bias, const void* w1, const void* w3,
                                 const void* w2, const void* ws1, const void* ws3,
                                 const void* ws2, void* out, int32_t* topk_idx,
                                 float* topk_gate, void* stream);

/* Bytes of moe_forward_noalloc's static scratch array (64 MiB). */
size_t moe_noalloc_scratch_bytes(void);

/* ---- Training side: forward that saves what the backward needs, and the
 * backward itself. ---------------------------------------------------------
 *
 * Objective whose gradients moe_backward returns:
 *
 *   Lambda = sum_{t,j} dout[t,j] * out[t,j]  +  alpha * L_bal
 *
 * dout is the upstream gradient dLoss/dout.  L_bal is the expert-level
 * balance loss of "DeepSeekMoE 深度解读报告" (sections 2.5 and 3.2), which
 * takes, over the batch, each expert's hit rate and mean gate score; the
 * pages print no formula, and the reading here is
 *
 *   f_e = E * n_e / (K * T)        n_e = rows routed to expert e
 *   P_e = (1/T) * sum_t s[t,e]     s = the full score vector of the gate
 *                                  (softmax or sigmoid, before renormalising)
 *   L_bal = sum_e f_e * P_e        (f_e held constant: a count has no gradient)
 *
 * The top-K choice is piecewise constant, so gradients reach the affinities
 * only through the kept gates and, via L_bal, through every score.  The
 * per-expert bias is a fixed input (no gradient).
 *
 * Bytes of the training state moe_forward_train writes and moe_backward
 * reads (the forward's workspace plus every expert's score of every token,
 * per-row gates, and the pre-activations Z = [W1 x | W3 x] of every row,
 * bf16).  0 for an invalid shape. */
size_t moe_train_state_size(const moe_shape_t* shape);

/* Bytes of device workspace moe_backward needs (dZ = [dA | dB] and g * H of
 * every row, the gate-gradient partials, the affinity gradients, the
 * per-row input gradients and work lists).  0 for an invalid shape. */
size_t moe_backward_workspace_size(const moe_shape_t* shape);

/* The layer forward of moe_forward (bit-identical out, topk_idx,
 * topk_gate), with the training state written to `state`
 * (moe_train_state_size() bytes, 256-byte aligned, caller-owned; keep it
 * unchanged until the matching moe_backward).  balance_stats (fp32 [2E + 1]
 * or NULL): f_e for e < E, P_e at E + e, L_bal at 2E (0 when K == 0).
 * Errors as for moe_forward, with the state in place of the workspace. */
moe_status_t moe_forward_train(const moe_shape_t* shape, const void* x, const void* centroids,
                               const float* expert_bias, const void* w1, const void* w3,
                               const void* w2, const void* ws1, const void* ws3,
                               const void* ws2, void* out, int32_t* topk_idx, float* topk_gate,
                               float* balance_stats, void* state, size_t state_bytes,
                               void* stream);

/* Backward of the layer for upstream gradient dout (bf16 [T, d]) and
 * balance factor alpha >= 0, from the state of a moe_forward_train call
 * with the same shape, x, centroids, bias and weights (not re-checked).
 * Per row r (token t, routed gate g_r, 1 for a shared expert), with
 * A = W1 x, B = W3 x, H = silu(A) B:
 *
 *   dgate_r = <dout[t], W2 H>             (computed as <W2^T dout[t], H>)
 *   dH = g_r W2^T dout[t],  dA = dH B silu'(A),  dB = dH silu(A)
 *   dx[t] += W1^T dA + W3^T dB;  dW2 += g_r dout[t] H^T;
 *   dW1 += dA x[t]^T;  dW3 += dB x[t]^T
 *
 * then gate -> score -> affinity for every token (through the
 * renormalisation and the softmax or sigmoid of the shape's flags, plus
 * alpha * f_e / T on every score from L_bal), dx += dL C, dC = dL^T x, and
 * dx += dout (the residual, unless MOE_FLAG_NO_RESIDUAL).
 *
 *   dx          bf16 [T, d]
 *   dw1, dw3    bf16 [E, I, d];  dw2 bf16 [E, d, I]   (NULL iff K == 0;
 *               every expert is written, untouched ones with zeros)
 *   dws1, dws3  bf16 [Ks, Is, d]; dws2 bf16 [Ks, d, Is] (NULL iff Ks == 0)
 *   dC          fp32 [E, d]      (NULL iff K == 0)
 *   dgate       fp32 [T, K] or NULL: d Lambda / d gate of each kept expert
 *   workspace   moe_backward_workspace_size() bytes, 256-byte aligned
 *
 * Arithmetic: bf16 MFMA with fp32 accumulation; dZ, g * H, the affinity
 * gradients and each row's dx contribution stored as bf16; dx summed per
 * token in fp32 in a fixed order and rounded once.  Bit-identical from run
 * to run.  Errors: as moe_forward (MOE_ERR_WORKSPACE for a short state or
 * workspace, MOE_ERR_SHAPE also for alpha < 0 or not finite). */
moe_status_t moe_backward(const moe_shape_t* shape, const void* x, const void* centroids,
                          const void* w1, const void* w3, const void* w2, const void* ws1,
                          const void* ws3, const void* ws2, const void* dout, float alpha,
                          const void* state, size_t state_bytes, void* dx, void* dw1, void* dw3,
                          void* dw2, void* dws1, void* dws3, void* dws2, float* dC,
                          float* dgate, void* workspace, size_t workspace_bytes, void* stream);

/* Routing only: affinities, softmax (or the flags' gate), top-K
 * ("DeepSeekMoE 深度解读报告", section 3.1).  Writes topk_idx [T, K] and topk_gate [T, K] (both
 * required).  The workspace needs moe_route_workspace_size() bytes (routing
 * scratch only, far less than a forward's).  K must be >= 1. */
moe_status_t moe_route(const moe_shape_t* shape, const void* x, const void* centroids,
                       const float* expert_bias, int32_t* topk_idx, float* topk_gate,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* moe_status_string(moe_status_t status);

/* Benchmark instrumentation (not part of the layer's computation).
 *
 * moe_profile_begin(max_calls): the next max_calls (1..100000) forward or
 * backward calls record a HIP event before and after each kernel they
 * launch, on the call's stream.  It creates 36*max_calls HIP events
 * (host-side runtime objects; no device memory).  Errors: MOE_ERR_SHAPE for a bad count,
 * MOE_ERR_NO_DEVICE / MOE_ERR_DEVICE_ARCH as for moe_forward, MOE_ERR_HIP if
 * event creation fails.
 *
 * moe_profile_end(ms, launches, n_slots): waits for the recorded events and
 * writes, for kernel slot k < n_slots, the summed duration in milliseconds
 * (ms[k], host array) and the number of timed launches (launches[k], host
 * array; either pointer may be NULL), then releases the events and stops
 * recording.  MOE_ERR_NULL if no recording is active, MOE_ERR_HIP if an event
 * could not be read.  Slots: 0 router, 1 router_tickets (small batches only), 2 perm_scan,
 * 3 perm_scatter, 4 gemm_gate_up, 5 gemm_down, 6 combine; moe_backward's
 * 7 bwd_lists, 8 bwd_dh, 9 bwd_router, 10 bwd_dx_router, 11 bwd_dx,
 * 12 bwd_dx_combine, 13 bwd_dw2, 14 bwd_dw13, 15 bwd_dc (a backward call
 * counts as a call); with MOE_FLAG_ACT8 16 act8_x, 17 act8_h (the
 * quantisation of x and of h's routed rows) (moe_profile_slot_name gives
 * the name, "" past the end).
 *
 * One process-wide recorder: not thread-safe; do not record from several
 * host threads at once. */
moe_status_t moe_profile_begin(int32_t max_calls);

/* moe_profile_begin_slots(max_calls, slot_mask): as moe_profile_begin, but
 * only the kernel slots whose bit is set in slot_mask (bit k = slot k, the
 * slot numbers below) are recorded; the others report 0 ms and 0 launches.
 * Each recorded kernel adds two event records to the stream (a few
 * microseconds each), so a timing run records only the kernel it needs.
 * Errors as moe_profile_begin, and MOE_ERR_SHAPE for an empty mask or bits
 * past the last slot. */
moe_status_t moe_profile_begin_slots(int32_t max_calls, uint32_t slot_mask);
moe_status_t moe_profile_end(float* ms, int32_t* launches, int32_t n_slots);
const char* moe_profile_slot_name(int32_t slot);

/* moe_profile_stream_read(buf, bytes, stream): enqueue one pass of 16-byte
 * loads over `bytes` of device memory at `buf` (caller-owned, 16-byte
 * aligned, contents irrelevant, never written), on `stream`.  Timed by the
 * caller, it gives the device's practical HBM read rate, the ceiling that the
 * HBM-bound kernels are compared with beside the nominal peak.  Errors:
 * MOE_ERR_NULL, MOE_ERR_SHAPE (bytes not a positive multiple of 32768),
 * MOE_ERR_ALIGN, MOE_ERR_NO_DEVICE / MOE_ERR_DEVICE_ARCH, MOE_ERR_HIP. */
moe_status_t moe_profile_stream_read(const void* buf, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
