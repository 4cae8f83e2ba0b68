/*
 * fwd.h — C ABI of the MI355X (gfx950) prefill forward library, libfwd.so.
 *
 * The library computes the forward pass of a decoder-only transformer over a
 * batch of prompts ("N7 · model/forward-parity", introduction and Theorem 1):
 * scaled embedding lookup, then per layer RMSNorm, the Q/K/V/O projections,
 * RoPE, causal grouped-query attention with an optional sliding window, the
 * SwiGLU feed-forward and the residual adds, with pre-norm or sandwich-norm
 * placement; then the final norm, the tied LM head with an optional final-logit
 * softcap ("pegainfer issue #878", Description and Proposed Plan), and the
 * per-position argmax. Projections are Y = X·Wᵀ with W stored [out, in]
 * ("N9 · metalgemm", Theorem 1).
 *
 * Conventions for every entry point:
 *  - Plain C types only. Pointers documented as "device" point to HIP device
 *    memory; "host" pointers to ordinary host memory.
 *  - All GPU work is enqueued on the hip stream passed in (NULL = the null
 *    stream). Functions return once the work is enqueued, except where stated.
 *  - Return value: FWD_OK (0) or a negative FWD_E_* code; the message of the
 *    last failure on the calling thread is available from fwd_last_error().
 *  - Nothing aborts and nothing falls back to a CPU computation: with no usable
 *    gfx950 device every compute entry point returns FWD_E_UNAVAILABLE.
 *  - bf16 means the 16-bit brain floating-point format (upper half of an IEEE
 *    binary32); all accumulation is in fp32.
 */
#ifndef FWD_H_
#define FWD_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define FWD_OK 0
#define FWD_E_CONFIG (-1)      /* invalid or unsupported geometry / numerics        */
#define FWD_E_WEIGHTS (-2)     /* a required weight pointer is NULL                 */
#define FWD_E_TOKEN_RANGE (-3) /* a token id lies outside [0, vocab)                */
#define FWD_E_TOO_LARGE (-4)   /* B*S exceeds the model's max_tokens                */
#define FWD_E_NONFINITE (-5)   /* a logit came out NaN or infinite                  */
#define FWD_E_HIP (-6)         /* a HIP runtime call failed (message has details)   */
#define FWD_E_UNAVAILABLE (-7) /* no usable gfx950 device                           */
#define FWD_E_ARG (-8)         /* bad argument (NULL handle, negative size, ...)    */

/* ---- enumerations ---- */
#define FWD_DTYPE_F32 0
#define FWD_DTYPE_BF16 1
#define FWD_EMBED_SCALE_NONE 0
#define FWD_EMBED_SCALE_BF16_SQRT_HIDDEN 1 /* sqrt(hidden) rounded to bf16 (issue #878) */
#define FWD_NORM_PRE 0
#define FWD_NORM_SANDWICH 1 /* RMSNorm on the sublayer input and on its output */
#define FWD_LAYER_GLOBAL 0
#define FWD_LAYER_LOCAL 1   /* sliding-window attention layer                 */
#define FWD_FFN_SILU 0      /* a = silu(g) * u (SwiGLU)                        */
#define FWD_FFN_GELU_TANH 1 /* a = gelu(g) * u, GELU in its tanh form          */
#define FWD_ROPE_NONE 0
#define FWD_ROPE_LLAMA3 1   /* llama3 frequency bands                          */
#define FWD_ROPE_LONGROPE 2 /* phi3 longrope per-frequency factors             */
#define FWD_FFN_DENSE 0     /* the layer's feed-forward is the dense gated FFN */
#define FWD_FFN_MOE 1       /* mixture of experts                              */

/*
 * Model description ("pegainfer issue #878", Proposed Plan: one typed config,
 * geometry derived from it, softcap validated positive at parse).
 *  n_layers, hidden (H), n_heads (Hq), n_kv_heads (Hkv, divides Hq),
 *  head_dim (D, even), ffn (F), vocab (V)
 *  rms_eps              RMSNorm epsilon (> 0)
 *  rope_theta           RoPE base (> 1); rotate-half pairs (k, k + D/2)
 *  embed_scale_mode     FWD_EMBED_SCALE_*
 *  final_logit_softcap  0 = off; otherwise z <- c * tanh(z / c); c < 0 or NaN is FWD_E_CONFIG
 *  sliding_window       W > 0: a local layer's query i sees keys j with 0 <= i - j < W
 *  layer_kind           host array of n_layers FWD_LAYER_* values, read during
 *                       fwd_create only; NULL = every layer global
 *  norm_placement       FWD_NORM_*
 *  dtype                FWD_DTYPE_BF16 (weights and GEMM operands bf16) or
 *                       FWD_DTYPE_F32 (everything fp32)
 *  max_tokens           largest B*S a later fwd_prefill may request; sizes the
 *                       workspace that fwd_create allocates
 *
 * Architecture variants ("N7 · model/forward-parity", Theorem statement names these
 * family axes: qwen3 QK-norm, gemma3 local/global attention, llama3 rope scaling,
 * phi3 longrope; the pages give no formulas, so each follows its family's published
 * definition). Zero-initialised fields give the plain model above.
 *  qk_norm              1: each q and k head is RMS-normalised over its head_dim
 *                       values (gains q_norm / k_norm, eps rms_eps) before RoPE
 *  norm_gain_offset     0: every RMSNorm scales by its gain w; 1: by (1 + w)
 *  ffn_act              FWD_FFN_*: the gate activation of the feed-forward
 *  rope_theta_local     RoPE base of local layers; 0 = rope_theta
 *  rope_scaling         FWD_ROPE_*. With base frequencies f_k = theta^(-2k/D):
 *    LLAMA3    wavelengths 2 pi / f_k below original_max_pos / high_freq_factor keep
 *              f_k, those above original_max_pos / low_freq_factor become f_k /
 *              factor, and in between t = (original_max_pos / wavelength -
 *              low) / (high - low) blends them as (1 - t) f_k / factor + t f_k
 *    LONGROPE  f_k = 1 / (e_k theta^(2k/D)) with e = long_factor when the sequence of
 *              the call (its last position + 1) exceeds original_max_pos, else
 *              short_factor; cos and sin are scaled by sqrt(1 + ln factor / ln
 *              original_max_pos) when factor > 1. A cached session keeps each key
 *              rotated as its own call rotated it.
 *  rope_factor, rope_low_freq_factor, rope_high_freq_factor, rope_original_max_pos
 *                       the parameters above (factor > 0; llama3: 0 < low < high)
 *  rope_short_factor, rope_long_factor
 *                       host arrays of head_dim / 2 positive floats (longrope), read
 *                       during fwd_create only
 *
 * Mixture of experts (the qwen3moe hybrid dense/sparse axis of the same Theorem
 * statement; the forward-parity intro lists the MoE FFN), bf16 only:
 *  n_experts            E (0 = dense everywhere; at most 256)
 *  n_experts_per_tok    k (1 .. min(8, E))
 *  moe_ffn              F_e, width of each expert's gated FFN (multiple of 32)
 *  moe_norm_topk        1: the k weights are renormalised to sum 1
 *  ffn_kind             host array of n_layers FWD_FFN_DENSE / FWD_FFN_MOE values, read
 *                       during fwd_create only; NULL = every layer MoE when n_experts > 0
 * A MoE layer's feed-forward output for a token is sum_j w_j FFN_{e_j}(n): e_1..e_k
 * are the experts with the k largest router logits n·W_routerᵀ (the softmax is
 * monotone; lowest index first on ties) and w_j their softmax probabilities over all E
 * experts, renormalised when moe_norm_topk. FFN_e is the gated FFN (ffn_act) with
 * expert e's matrices.
 *
 * Supported: bf16 needs head_dim in {64, 128, 256}; f32 needs head_dim <= 64;
 * hidden, Hq*D, Hkv*D and ffn multiples of 8 (bf16) or 4 (f32); bf16 additionally
 * needs hidden, Hq*D, Hkv*D and ffn multiples of 32 (its GEMM operands are stored in
 * 32-column tiles).
 */
typedef struct fwd_config {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps;
  float final_logit_softcap;
  double rope_theta;
  int32_t embed_scale_mode;
  int32_t sliding_window;
  const int32_t* layer_kind;
  int32_t norm_placement;
  int32_t dtype;
  int32_t max_tokens;
  /* architecture variants (appended; zero = off) */
  int32_t qk_norm;
  int32_t norm_gain_offset;
  int32_t ffn_act;
  double rope_theta_local;
  int32_t rope_scaling;
  float rope_factor;
  float rope_low_freq_factor;
  float rope_high_freq_factor;
  int32_t rope_original_max_pos;
  const float* rope_short_factor;
  const float* rope_long_factor;
  /* mixture of experts (appended; zero = dense) */
  int32_t n_experts;
  int32_t n_experts_per_tok;
  int32_t moe_ffn;
  int32_t moe_norm_topk;
  const int32_t* ffn_kind;
} fwd_config;

/*
 * Weights of one layer: device pointers, row-major W[out, in], element type
 * bf16 or f32 according to fwd_config.dtype (norm gains too).
 *  wq [Hq*D, H], wk [Hkv*D, H], wv [Hkv*D, H], wo [H, Hq*D],
 *  w_gate [F, H], w_up [F, H], w_down [H, F], *_norm [H].
 *  post_attn_norm / post_ffn_norm are read only for FWD_NORM_SANDWICH;
 *  q_norm / k_norm [D] only with qk_norm.
 *  MoE layers read router [E, H], expert_gate and expert_up [E, F_e, H] and
 *  expert_down [E, H, F_e] (each expert's matrix contiguous, row-major) instead of
 *  w_gate / w_up / w_down.
 */
typedef struct fwd_layer_weights {
  const void* attn_norm;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const void* ffn_norm;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* post_attn_norm;
  const void* post_ffn_norm;
  const void* q_norm;
  const void* k_norm;
  const void* router;
  const void* expert_gate;
  const void* expert_up;
  const void* expert_down;
} fwd_layer_weights;

/* embed [V, H] (also the tied LM head), final_norm [H]: device pointers;
 * layers: host array of n_layers entries. */
typedef struct fwd_weights {
  const void* embed;
  const void* final_norm;
  const fwd_layer_weights* layers;
} fwd_weights;

/*
 * Caller-owned device output buffers of one fwd_prefill; any may be NULL to skip it.
 *  logits [B, S, V] fp32 (after the softcap when it is on)
 *  hidden [L + 2, B, S, H] fp32: slot 0 = scaled embedding, slot l + 1 = the
 *         residual stream after layer l, slot L + 1 = final-norm output
 *         ("N7 · model/forward-parity", Theorem 1: one hidden slot per layer)
 *  argmax [B, S] int32: per-position argmax of the logits, lowest index on ties
 */
typedef struct fwd_outputs {
  float* logits;
  float* hidden;
  int32_t* argmax;
} fwd_outputs;

/* Element counts of the outputs, and bytes the library allocates for a model. */
typedef struct fwd_sizes {
  int64_t logits_elems;
  int64_t hidden_elems;
  int64_t argmax_elems;
  int64_t weight_bytes;
  int64_t workspace_bytes;
} fwd_sizes;

typedef struct fwd_model fwd_model;

/* 1 if a gfx950 device is visible and usable, else 0 ("N9 · metalgemm",
 * Theorem 2: Available()). Never fails. */
int fwd_available(void);

/*
 * Validate cfg, allocate the model on the current HIP device, and copy the
 * weights into library-owned HBM in the library's packed layout
 * ("N9 · metalgemm", Theorem 2: Upload / FwdConfig / FwdLayer / FwdFinalNorm).
 * The weight buffers are only read during this call (the copies run on
 * hip_stream and are complete when it returns), so the caller may free them
 * afterwards. The model keeps hip_stream for later fwd_prefill calls.
 * On success *out receives the handle (release with fwd_destroy).
 * Errors: FWD_E_ARG, FWD_E_CONFIG, FWD_E_WEIGHTS, FWD_E_HIP, FWD_E_UNAVAILABLE.
 */
int fwd_create(const fwd_config* cfg, const fwd_weights* w, void* hip_stream, fwd_model** out);

/*
 * Sizes of the outputs of a (B, S) prefill and of the model's own allocations
 * — the one source of truth for buffer sizes ("pegainfer issue #878", Proposed
 * Plan). Pure host computation; needs no device. Errors: FWD_E_ARG, FWD_E_CONFIG.
 */
int fwd_output_sizes(const fwd_config* cfg, int32_t B, int32_t S, fwd_sizes* out);

/*
 * Forward pass over B independent prompts of S tokens each (positions 0..S-1).
 * ids_host: host int32 [B, S]. Every id is checked against [0, vocab) on the
 * host before anything is uploaded ("pegainfer issue #878", Proposed Plan);
 * a bad id returns FWD_E_TOKEN_RANGE and enqueues nothing. B*S must not exceed
 * max_tokens (FWD_E_TOO_LARGE). S == 0 or B == 0 is a no-op.
 * Blocks until the work on the model's stream is finished, then returns
 * FWD_E_NONFINITE if any logit was NaN or infinite ("pegainfer issue #878",
 * Acceptance Criteria: non-finite values fail outright); outputs are then
 * unspecified. Calls on one model must not overlap.
 */
int fwd_prefill(fwd_model* m, const int32_t* ids_host, int32_t B, int32_t S, const fwd_outputs* out);

/*
 * Standalone projection Y[p, o] = sum_i X[p, i] * W[o, i] ("N9 · metalgemm",
 * Theorem 1: Weight.MatMul). X device [P, in], W device [out, in], both of
 * `dtype` (FWD_DTYPE_BF16 or FWD_DTYPE_F32); Y device fp32 [P, out]. fp32
 * accumulation. `in` must be a multiple of 8 (bf16) or 4 (f32).
 * bf16 products with few output tiles and a long `in` are cut into ranges of `in`
 * whose fp32 partial products are added in range order (deterministic: a call
 * repeats bit for bit); their partials live in device memory the call allocates
 * and frees in stream order on hip_stream, from a memory pool of its own that keeps
 * the memory for later calls.
 * Errors: FWD_E_ARG, FWD_E_UNAVAILABLE, FWD_E_HIP.
 */
int fwd_gemm(const void* X, const void* W, float* Y, int32_t P, int32_t in, int32_t out,
             int32_t dtype, void* hip_stream);

/*
 * fwd_gemm for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments,
 * the same kernels and the same result bit for bit, with no allocation of any kind.
 * The split partials of products that fwd_gemm cuts into ranges of `in` live in a
 * static device array of 16 MiB that every GPU the library runs on holds until the
 * process ends; a product whose partials need more returns FWD_E_TOO_LARGE and
 * computes nothing. The array is shared by every call on a GPU and keeps the last
 * call's partials (each call writes every partial it reads): calls that overlap on one
 * GPU race.
 * Errors: FWD_E_ARG, FWD_E_TOO_LARGE, FWD_E_UNAVAILABLE, FWD_E_HIP.
 */
int fwd_gemm_noalloc(const void* X, const void* W, float* Y, int32_t P, int32_t in, int32_t out,
                     int32_t dtype, void* hip_stream);

/*
 * Causal grouped-query attention alone, the operation inside each layer
 * ("N7 · model/forward-parity", introduction; "N9 · metalgemm", Theorem 1 op
 * chain): o[b,i,h,:] = sum_j softmax_j(q[b,i,h,:]·k[b,j,g,:] / sqrt(D)) v[b,j,g,:]
 * over keys j <= i (and i - j < window when window > 0), g = h / (Hq / Hkv).
 * Device buffers of `dtype`: q [B, S, Hq, D], k [B, S, Hkv, D],
 * v_t [B, Hkv, D, Sp] with Sp = S rounded up to a multiple of 8 (values
 * transposed, keys contiguous; the entries past S are read with weight exactly
 * zero, so they must be finite), o [B, S, Hq, D].
 * No RoPE is applied here. Errors: FWD_E_ARG, FWD_E_CONFIG, FWD_E_UNAVAILABLE, FWD_E_HIP.
 */
int fwd_attention(const void* q, const void* k, const void* v_t, void* o, int32_t B, int32_t S,
                  int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t window,
                  int32_t dtype, void* hip_stream);

/*
 * RMSNorm alone ("N7 · model/forward-parity", introduction):
 * y[r, i] = x[r, i] * w[i] / sqrt(mean_j x[r, j]^2 + eps).
 * x device fp32 [rows, H]; w device fp32 [H]; y device [rows, H] of `dtype`.
 * H must be a multiple of 4.
 * Errors: FWD_E_ARG, FWD_E_UNAVAILABLE, FWD_E_HIP.
 */
int fwd_rmsnorm(const float* x, const void* w, void* y, int32_t rows, int32_t hidden, float eps,
                int32_t dtype, void* hip_stream);

/*
 * Mixture-of-experts routing alone (the decision inside a MoE layer; see fwd_config):
 * for each of T rows of router logits [T, E] (device fp32), idx[t, j] (device int32
 * [T, k]) = the experts with the k largest logits, largest first, lowest index first
 * on ties; w[t, j] (device fp32 [T, k]) = their softmax probabilities over all E,
 * divided by their sum when norm_topk. 1 <= k <= min(8, E), E <= 256.
 * Errors: FWD_E_ARG, FWD_E_UNAVAILABLE, FWD_E_HIP.
 */
int fwd_moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t norm_topk, int32_t* idx, float* w,
                  void* hip_stream);

/*
 * Per-kernel timing of fwd_prefill with HIP events recorded on the model's stream
 * around every launch (off by default). Kernel classes:
 */
#define FWD_KERNEL_EMBED 0         /* scaled embedding gather                      */
#define FWD_KERNEL_NORM 1          /* RMSNorm, and the fused sandwich add + norm   */
#define FWD_KERNEL_QKV_ROPE 2      /* QKV projection with the RoPE epilogue        */
#define FWD_KERNEL_ATTENTION 3     /* causal GQA attention                         */
#define FWD_KERNEL_O_PROJ 4        /* output projection (+ residual add)           */
#define FWD_KERNEL_GATE_UP 5       /* gate/up projection with the SwiGLU epilogue  */
#define FWD_KERNEL_DOWN_PROJ 6     /* down projection (+ residual add)             */
#define FWD_KERNEL_LM_HEAD 7       /* tied LM head (+ softcap)                     */
#define FWD_KERNEL_ARGMAX 8        /* per-position argmax + non-finite check      */
#define FWD_KERNEL_V_TRANSPOSE 9   /* values transposed to keys-contiguous order  */
#define FWD_KERNEL_QK_NORM 10      /* QK-norm + RoPE pass (qk_norm models)        */
#define FWD_KERNEL_MOE_ROUTE 11    /* router product, top-k, permutation, gather  */
#define FWD_KERNEL_MOE_EXPERTS 12  /* grouped expert products                     */
#define FWD_KERNEL_MOE_COMBINE 13  /* weighted sum of the expert outputs          */
#define FWD_KERNEL_CLASSES 14
/* enable != 0 turns timing on and clears the accumulated totals; 0 turns it off. */
int fwd_set_timing(fwd_model* m, int32_t enable);
/* Accumulated milliseconds and launch count of one kernel class since the last
 * fwd_set_timing(m, 1). Errors: FWD_E_ARG. */
int fwd_get_timing(const fwd_model* m, int32_t kernel_class, double* total_ms, int64_t* launches);

/* Release a model and everything it allocated (waits for its stream first).
 * NULL is a no-op ("N9 · metalgemm", Theorem 1: Free / Reset reclaim the table).
 * Destroy the model's sessions first. */
void fwd_destroy(fwd_model* m);

/*
 * ---- Cached sessions: prefill into a KV cache, then greedy decode ----
 * ("N7 · model/forward-parity", Theorem 1: a cached session's prefill reproduces the
 * cacheless forward's last-position logits, and the greedy continuation ids match
 * token for token; "N9 · metalgemm", Theorem 1: argmax-exact and cosine-close at every
 * prefill and greedy step.)
 *
 * A session borrows its model (destroy the session first) and owns, per layer, a
 * key and a value cache of max_batch x n_kv_heads x max_seq x head_dim elements of
 * the model's dtype, plus a RoPE table for max_seq positions. Work runs on the
 * model's stream. Calls on one model (through any of its sessions or fwd_prefill)
 * must not overlap; the model's workspace is shared.
 * Errors: FWD_E_ARG, FWD_E_TOO_LARGE (max_batch above the model's max_tokens),
 * FWD_E_CONFIG (more than 16 query heads per kv head), FWD_E_HIP.
 */
typedef struct fwd_session fwd_session;
int fwd_session_create(fwd_model* m, int32_t max_batch, int32_t max_seq, fwd_session** out);

/*
 * Start the session over B prompts of S tokens each (host int32 [B, S], positions
 * 0..S-1): the same forward pass and outputs as fwd_prefill, and every layer's
 * rotated keys and values are stored in the cache. Replaces whatever the session
 * held; afterwards it holds B sequences of length S.
 * Errors: as fwd_prefill; FWD_E_TOO_LARGE if B > max_batch, S > max_seq or
 * B*S > max_tokens. On an error the session is left empty.
 */
int fwd_session_prefill(fwd_session* s, const int32_t* ids_host, int32_t B, int32_t S, const fwd_outputs* out);

/*
 * Extend every sequence by one token: ids_host is host int32 [B] (B of the last
 * prefill), placed at position len (the current length). Its keys and values are
 * appended to the cache and attention runs over positions 0..len (or the last
 * `sliding_window` of them on local layers). Outputs as for a prefill with S = 1:
 * logits [B, V] fp32, hidden [n_layers + 2, B, H] fp32, argmax [B]; any may be NULL.
 * Errors: FWD_E_ARG (no prefill yet), FWD_E_TOO_LARGE (len == max_seq),
 * FWD_E_TOKEN_RANGE, FWD_E_NONFINITE, FWD_E_HIP.
 */
int fwd_session_decode(fwd_session* s, const int32_t* ids_host, const fwd_outputs* out);

/* Current length of the session's sequences (0 before a prefill; -1 for NULL). */
int32_t fwd_session_length(const fwd_session* s);

/* Release a session's caches (waits for the model's stream). NULL is a no-op. */
void fwd_session_destroy(fwd_session* s);

/* Message of the last failure on the calling thread ("" if none). The pointer
 * stays valid until the next call into the library on that thread. */
const char* fwd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FWD_H_ */
