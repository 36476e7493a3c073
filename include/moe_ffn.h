/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) mixture-of-experts FFN library.
 *
 * The library computes the MoE feed-forward layer of a decoder block, in
 * the op order that hf2q's qwen35/gpu_ffn.rs states in its module header
 * ("MoE FFN op order"):
 *
 *   1. router logits      l[t,e] = x[t,:] . router[e,:] (+ router_bias[e])
 *   2. routing            softmax over the E logits (or a sigmoid per
 *                         logit, moe_gating), the top_k experts by score
 *                         (ties: lower expert index first), optionally
 *                         times a per-expert scale, weights renormalised
 *                         over the selected experts (hf2q
 *                         softmax_topk_renorm_cpu), times routed_scale
 *   3. routed experts     for each selected expert e of token t:
 *                         h = act(gate[e] x) * (up[e] x),  y = down[e] h
 *                         (act = SiLU, or the tanh form of GELU used by
 *                         mlx-native's moe_dispatch.rs)
 *   4. combine            out[t] = sum_j w[t,j] * y[t,j]
 *   5. shared expert      out[t] += sigmoid(x . shared_gate_inp)
 *                                   * shared_down(silu(shared_gate x) *
 *                                                 (shared_up x))
 *
 * Two optional ends (moe_desc.pre_norm, the residual of moe_ffn_forward):
 * x may first be replaced by RMSNorm(x) * norm_weight, and a residual may
 * be added to out.
 *
 * Layouts are row-major with the last index contiguous; weight matrices are
 * [out, in] (y = W x), the stacked-expert layout of hf2q's
 * MoeFfnWeightsGpu and of ferrum-kernels' validate_participant bindings.
 * Routed expert weights are stacked densely: expert e of gate/up starts at
 * element e*I*H, expert e of down at e*H*I.
 *
 * Memory: every pointer argument is caller-owned device memory (hipMalloc
 * or equivalent), except the moe_desc / moe_weights structs and the
 * `bytes` out-parameter, which are host memory read (or written) during
 * the call only.  The library allocates nothing per call: scratch comes
 * from the caller's workspace, sized by moe_workspace_size (the affine
 * workspace formula of ferrum-kernels' MoeWorkspaceLayout).
 *
 * Workspace: its first MOE_WORKSPACE_ZERO_BYTES bytes hold completion
 * counters that every call leaves at zero when its work ends.  Fill them
 * with zeros once, after allocating the workspace and before its first
 * use; after that, reuse it as it is.  Calls sharing one workspace must
 * not overlap in time (same stream, or ordered by events).
 *
 * Streams: calls enqueue work on `stream` (a hipStream_t; NULL = the
 * default stream) and return without synchronising.  Buffers must stay
 * valid until that work completes.
 *
 * Errors: all validation happens on the host before the first enqueue; a
 * call that returns anything but MOE_OK has enqueued nothing and written
 * nothing (the error-path contract of mlx-native's rejects_size_mismatch
 * test).  moe_last_error() then returns a thread-local message.  A HIP
 * launch failure after enqueueing started returns MOE_HIP_ERROR.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FFN_ABI_VERSION 8

/* Leading workspace bytes that must be zero before a workspace's first use. */
#define MOE_WORKSPACE_ZERO_BYTES 256

/* Limits (ferrum-kernels moe.rs route dispatch: at most 256 experts and
 * 32 experts per token). */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOP_K 32

typedef enum moe_status {
  MOE_OK = 0,
  MOE_INVALID_ARGUMENT = 1,    /* null pointer, bad size, k > E, ...       */
  MOE_UNSUPPORTED = 2,         /* valid but not implemented (alignment...) */
  MOE_WORKSPACE_TOO_SMALL = 3, /* ws_bytes < moe_workspace_size(...)       */
  MOE_HIP_ERROR = 4            /* a HIP launch failed                      */
} moe_status;

typedef enum moe_weight_format {
  MOE_WEIGHTS_F32 = 0,
  MOE_WEIGHTS_BF16 = 1,
  /* affine 4-bit, groups of 32 along K: w = code * scale + min, the
   * (scale, bias) form hf2q's dispatch_moe_id_routed passes to its affine
   * quantized matmul.  codes: uint8 [E, N, K/2], element 2i in the low
   * nibble of byte i, element 2i+1 in the high nibble; scales and mins:
   * IEEE fp16 [E, N, K/32]. */
  MOE_WEIGHTS_U4_G32 = 2
} moe_weight_format;

typedef enum moe_activation {
  MOE_ACT_SILU = 0,       /* z / (1 + exp(-z))                              */
  MOE_ACT_GELU_TANH = 1   /* 0.5 z (1 + tanh(0.7978845608 (z + 0.044715 z^3))) */
} moe_activation;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Routing scores from the router logits l (ferrox-models decoder.rs: the
 * gating function of the MoE config; its dense-layer note states that
 * sigmoid gating with renormalisation divides a selected score by the sum
 * of the selected scores).  Either way the k experts with the largest
 * scores are selected, the lower expert index first among equal scores;
 * both scores are increasing in l, so this is the order of the logits. */
typedef enum moe_gating {
  MOE_GATING_SOFTMAX = 0,  /* p = softmax(l) over all E experts           */
  MOE_GATING_SIGMOID = 1   /* p_e = 1 / (1 + exp(-l_e)), each on its own   */
} moe_gating;

/* Shape and format attributes (ferrum-kernels MoeAttributes). */
typedef struct moe_desc {
  int32_t hidden;              /* H                                          */
  int32_t intermediate;        /* I, routed experts                          */
  int32_t num_experts;         /* E, 1..256                                  */
  int32_t top_k;               /* k, 1..min(E, 32)                           */
  int32_t activation;          /* moe_activation (routed experts)            */
  int32_t weight_format;       /* moe_weight_format (routed and shared)      */
  int32_t act_dtype;           /* moe_dtype of x                             */
  int32_t router_dtype;        /* moe_dtype of router and shared_gate_inp    */
  int32_t normalize_topk;      /* 1: renormalise the k weights; 0: raw scores */
  int32_t has_shared_expert;   /* 0 or 1                                     */
  int32_t shared_intermediate; /* Is (ignored without a shared expert)       */
  int32_t group_size;          /* 32 for MOE_WEIGHTS_U4_G32, else ignored    */
  int32_t gating;              /* moe_gating                                 */
  float routed_scale;          /* every routing weight is multiplied by it
                                  (llama.cpp's w_scale, which ferrox-models
                                  names in gpt_oss_ffn); finite, 1 for none */
  int32_t pre_norm;            /* 1: the layer runs on RMSNorm(x) (the
                                  pre-FFN norm of ferrox-models' decoder
                                  step), x[t] / sqrt(mean(x[t]^2) + norm_eps)
                                  * norm_weight, rounded to act_dtype;
                                  0: on x as given                          */
  float norm_eps;              /* > 0 when pre_norm, else ignored            */
  int32_t out_dtype;           /* moe_dtype of out: MOE_F32, the fp32 output
                                  of mlx-native's weighted-sum accumulator
                                  and of hf2q's layer (MOE_BF16 is
                                  UNSUPPORTED: no reduced-precision output
                                  is built)                                 */
} moe_desc;

typedef struct moe_u4_matrix {
  const uint8_t* codes;    /* [E, N, K/2]  */
  const uint16_t* scales;  /* fp16 bits [E, N, K/32] */
  const uint16_t* mins;    /* fp16 bits [E, N, K/32] */
} moe_u4_matrix;

/* Device pointers to the layer's weights. */
typedef struct moe_weights {
  const void* router;          /* [E, H], router_dtype                       */
  const float* router_bias;    /* [E] f32, or NULL                           */
  const void* gate;            /* [E, I, H] f32/bf16 (NULL for u4)           */
  const void* up;              /* [E, I, H]                                  */
  const void* down;            /* [E, H, I]                                  */
  moe_u4_matrix gate_u4;       /* used when weight_format == U4_G32          */
  moe_u4_matrix up_u4;
  moe_u4_matrix down_u4;
  const void* shared_gate_inp; /* [H], router_dtype (shared expert only)     */
  const void* shared_gate;     /* [Is, H], f32/bf16                          */
  const void* shared_up;       /* [Is, H]                                    */
  const void* shared_down;     /* [H, Is]                                    */
  const float* norm_weight;    /* [H] f32 (pre_norm only)                    */
  /* Optional, bf16 weights only: the same expert weights in the packed
   * layout moe_pack_weights writes.  When the prefill GEMMs stream weight
   * tiles (bf16 weights and activations, many routes per expert) they read
   * these instead of gate/up/down, as contiguous 32 KB blocks.  The
   * row-major pointers above stay required (the other paths read them).
   * gate_up_packed and shared_gate_up_packed are used together or not at
   * all, and so are down_packed and shared_down_packed; NULL: not used.  */
  const void* gate_up_packed;
  const void* down_packed;
  const void* shared_gate_up_packed;
  const void* shared_down_packed;
  /* [E] f32, 4-byte aligned, or NULL: a learned per-expert scale on the
   * routing weights (mlx-native moe_dispatch.rs, moe_gather_topk_weights_
   * encode: gather the top-k experts and their scores, apply
   * per_expert_scale, renormalise).  Selection looks at the scores alone;
   * then selected expert e's score p is replaced by p * expert_scale[e],
   * and the renormalisation (normalize_topk) divides by the sum of the
   * scaled scores.  routed_scale applies after that.  With
   * renormalisation, scales whose scaled sum is zero for a token give
   * non-finite weights; positive scales never do.  NULL: all ones. */
  const float* expert_scale;
} moe_weights;

/* ABI version (MOE_FFN_ABI_VERSION of the built library). */
int32_t moe_abi_version(void);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* moe_last_error(void);

/*
 * moe_workspace_size: bytes of scratch a call with `num_tokens` tokens
 * needs.  The size is affine in num_tokens (fixed part + per-token part),
 * as ferrum-kernels' workspace formula is.  Host only; enqueues nothing.
 * Errors: MOE_INVALID_ARGUMENT for a bad descriptor, num_tokens < 0 or a
 * NULL `bytes`.
 */
moe_status moe_workspace_size(const moe_desc* desc, int64_t num_tokens,
                              size_t* bytes);

/*
 * moe_route: steps 1-2 plus the expert grouping of the routes.
 *
 *   x              [T, H] act_dtype
 *   topk_ids       [T, k] int32 out: slot j holds the j-th most probable
 *                  expert (lower index first among equal probabilities)
 *   topk_w         [T, k] f32 out: routing weights (sum to routed_scale per
 *                  token when normalize_topk)
 *   expert_counts  [E] int32 out or NULL: routes that chose each expert
 *   expert_offsets [E+1] int32 out or NULL: exclusive prefix sum of counts
 *   route_perm     [T*k] int32 out or NULL: the flat routes r = t*k + j
 *                  grouped by expert, stable in r (the stable argsort of the
 *                  flat expert ids that DS4Server's gather_sort builds):
 *                  route_perm[expert_offsets[e] + i] is the i-th route,
 *                  in increasing r, that chose expert e.
 *   ws, ws_bytes   workspace, at least moe_workspace_size(desc, T) bytes
 *
 * Only weights->router, weights->router_bias, weights->expert_scale and
 * (with a shared expert) weights->shared_gate_inp are read.  T = 0 is a
 * no-op.
 */
moe_status moe_route(const moe_desc* desc, int64_t num_tokens, const void* x,
                     const moe_weights* weights, int32_t* topk_ids,
                     float* topk_w, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* route_perm, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * moe_ffn_forward: the whole layer, steps 1-5.
 *
 *   x            [T, H] act_dtype
 *   out          [T, H] f32 out (the f32 accumulator/output convention of
 *                mlx-native's moe_weighted_sum_seq)
 *   residual     [T, H] f32 or NULL: when given, out = layer(x) + residual,
 *                added in the kernel that writes out (hf2q folds the
 *                residual into its final weighted reduce the same way).
 *                It may be `out` itself (out += layer(x)).
 *   topk_ids_out [T, k] int32 out or NULL (as in moe_route)
 *   topk_w_out   [T, k] f32 out or NULL
 *   ws, ws_bytes workspace, at least moe_workspace_size(desc, T) bytes
 *
 * `out` must not alias x, the weights or the workspace.  T = 0 is a no-op.
 * MOE_UNSUPPORTED when hidden > 16384 unless the call takes the bf16 MFMA
 * path (bf16 weights and activations, T > 32, hidden, intermediate and
 * shared_intermediate multiples of 64): the decode kernels keep a route's
 * activation row in LDS.
 */
moe_status moe_ffn_forward(const moe_desc* desc, int64_t num_tokens,
                           const void* x, const moe_weights* weights,
                           float* out, const float* residual,
                           int32_t* topk_ids_out, float* topk_w_out,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * moe_ffn_forward_noalloc: moe_ffn_forward without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * scratch comes from a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, held until the process ends; the call
 * itself allocates nothing.  Arguments, results and errors are those of
 * moe_ffn_forward, plus MOE_UNSUPPORTED when the call needs more scratch
 * than the array holds (moe_workspace_size(desc, num_tokens) >
 * MOE_NOALLOC_SCRATCH_BYTES: decode shapes and small prefill batches fit).
 * All calls on one GPU share its array: calls that overlap in time on one
 * GPU (different streams not ordered by events, or different threads)
 * race and give undefined results.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_ffn_forward_noalloc(const moe_desc* desc, int64_t num_tokens,
                                   const void* x, const moe_weights* weights,
                                   float* out, const float* residual,
                                   int32_t* topk_ids_out, float* topk_w_out,
                                   void* stream);

/*
 * Backward of the routing-weighted combine (mlx-native moe_dispatch.rs,
 * moe_weighted_sum_seq and its two backward kernels).  Forward:
 * out[t,d] = sum_j w[t,j] * y[t,j,d].  Gradients, given dout = dL/dout:
 *
 *   dy[t,j,d] = w[t,j] * dout[t,d]
 *   dw[t,j]   = sum_d y[t,j,d] * dout[t,d]
 *
 *   w    [T, k] f32;   y [T, k, H] f32;   dout [T, H] f32
 *   dy   [T, k, H] f32 out, or NULL to skip it
 *   dw   [T, k] f32 out, or NULL to skip it
 *
 * All f32 device memory, 16-byte aligned; H a multiple of 4; k in 1..32.
 * Outputs must not alias inputs.  T = 0 is a no-op.
 */
moe_status moe_weighted_sum_backward(int64_t num_tokens, int32_t top_k, int32_t hidden,
                                     const float* w, const float* y, const float* dout,
                                     float* dy, float* dw, void* stream);

/*
 * Backward of the gated activation h = act(g) * u (mlx-native
 * moe_dispatch.rs, moe_swiglu_seq backward; act = SiLU or the tanh GELU of
 * moe_activation), one fused pass:
 *
 *   dg = dh * u * act'(g)
 *   du = dh * act(g)
 *
 *   gate_up  [R, 2I] f32: row r holds g (columns 0..I-1) then u (I..2I-1)
 *   dh       [R, I] f32
 *   d_gate_up[R, 2I] f32 out, the same layout (dg, then du)
 *
 * R = rows (routes); 16-byte aligned; I a multiple of 4.  R = 0 is a no-op.
 */
moe_status moe_glu_backward(int64_t rows, int32_t intermediate, int32_t activation,
                            const float* gate_up, const float* dh, float* d_gate_up,
                            void* stream);

/*
 * Packed expert weights: a layout of the bf16 expert weights for the prefill
 * grouped GEMMs.  DS4Server's qwen_mtplx.rs (its SwitchGLU weights) already
 * offers gate and up either as separate [E, I, H] matrices or fused into one
 * [E, 2I, H]; this layout goes further, for the way these GEMMs read weights.
 * They stream weight tiles 64 K-elements at a time; the packed layout stores
 * each tile's K-step as one contiguous 32 KB block, a sequential run instead
 * of 256 rows of 128 bytes.  The arithmetic, and so every result, is
 * unchanged.
 *
 * Layout (bf16 elements, 16-byte chunks): block (t, s) of an expert holds
 * K-elements 64s .. 64s+63 of its weight tile t as 256 rows of 128 bytes.
 * Gate/up tiles cover 128 features: row r < 128 is gate feature 128t + r,
 * row r >= 128 up feature 128t + r - 128 (t < ceil(I/128)).  Down tiles cover
 * 256 outputs: row r is output 256t + r (t < ceil(H/256)); its K is I.  Chunk
 * c of row r (elements 64s + 8c .. 64s + 8c + 7) is stored at chunk slot
 * c ^ ((r >> 1) & 7) of the row.  Rows past the matrix are zero.  An expert's
 * blocks are ordered t * (K/64) + s; experts are consecutive.  The shared
 * expert is packed the same way with Is for I.
 *
 * moe_packed_weight_bytes: the four arrays' sizes (0 for the shared expert's
 * when there is none).  Any output pointer may be NULL.  Host only.  Errors:
 * MOE_INVALID_ARGUMENT for a bad descriptor; MOE_UNSUPPORTED unless the
 * weights are bf16, hidden, intermediate and shared_intermediate are
 * multiples of 64, and one expert's packed matrix fits in 4 GiB.
 *
 * moe_pack_weights: enqueues the packing of weights->gate/up/down (and the
 * shared expert's) into the caller's device arrays, 16-byte aligned, of the
 * sizes above, on `stream`.  Reads only those weights; the destinations must
 * not overlap them.  Errors: as above, plus MOE_INVALID_ARGUMENT for a NULL
 * source or destination and MOE_UNSUPPORTED for a misaligned one.
 */
moe_status moe_packed_weight_bytes(const moe_desc* desc, size_t* gate_up_bytes,
                                   size_t* down_bytes, size_t* shared_gate_up_bytes,
                                   size_t* shared_down_bytes);
moe_status moe_pack_weights(const moe_desc* desc, const moe_weights* weights,
                            void* gate_up_packed, void* down_packed,
                            void* shared_gate_up_packed, void* shared_down_packed,
                            void* stream);

/*
 * Kernel timing, for measurement.  While enabled, every kernel the library
 * launches is bracketed by a pair of hipEvents recorded on the call's
 * stream.  moe_timing_read synchronises those events and returns, per
 * kernel name (at most `max_entries`), the number of launches and the
 * summed event-to-event milliseconds since the last reset; it returns the
 * number of entries written, or -1 on error.  Not for use under graph
 * capture.  Intended for benchmarks only.
 */
moe_status moe_timing_enable(int32_t enable);
int32_t moe_timing_read(char* names, int32_t name_stride, int64_t* launches,
                        double* total_ms, int32_t max_entries);
moe_status moe_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
