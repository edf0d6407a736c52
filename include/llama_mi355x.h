/*
 * llama_mi355x.h -- C ABI of the MI355X (gfx950) Llama 2 decoder forward.
 *
 * The library computes Transformer.forward(tokens, start_pos) of the Llama 2 reference
 * model as described in "Llama 2 Reference Implementation -- Administrator & Developer
 * Guide", section 8.4 "The model architecture in detail": token embedding, n_layers
 * pre-norm blocks (RMSNorm -> Q/K/V projection -> RoPE -> KV-cache append -> causal
 * grouped-query attention -> wo + residual; RMSNorm -> SwiGLU FFN -> w2 + residual), final
 * RMSNorm and the projection to vocabulary logits in fp32.  Greedy selection and the
 * token bookkeeping of the generate loop (section 8.5 "The generation loop in detail")
 * are separate calls so a caller can keep the whole loop on the device.
 *
 * Conventions for every entry point:
 *  - Pointers named d_* are device pointers (HBM of the current HIP device); everything
 *    else is host memory.  `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream); all device work is enqueued on it, asynchronously, in stream order.
 *  - Errors are returned, never raised: no entry point aborts.  Every precondition that
 *    can be checked on the host is checked before anything is launched; on error nothing
 *    is enqueued.  A failure of the HIP runtime (launch error, earlier asynchronous fault
 *    reported by the runtime) is returned as LLAMA_ERR_HIP.
 *  - A llama_ctx is not thread-safe; calls on one ctx must be ordered on one stream (or
 *    ordered by the caller across streams).
 *  - Token ids outside [0, vocab_size) are a precondition violation of the caller; the
 *    kernels clamp them into range rather than read out of bounds.  Checked mode (the
 *    environment variable LLAMA_MI355X_CHECK_TOKENS=1 when llama_init runs) checks them on
 *    the device: llama_prefill, llama_decode_step and llama_decode_step_noalloc then wait
 *    for the stream at the end of the call and return LLAMA_ERR_INVALID_ARG if any id of the
 *    call was out of range (the outputs are those of the clamped ids).  Meant for debugging:
 *    every call synchronises, and decode steps launch eagerly.
 */
#ifndef LLAMA_MI355X_H
#define LLAMA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LLAMA_MI355X_ABI_VERSION 1

typedef enum llama_status {
    LLAMA_OK = 0,
    LLAMA_ERR_INVALID_ARG = -1,  /* a precondition of the call does not hold */
    LLAMA_ERR_UNSUPPORTED = -2,  /* valid model, but a shape this library does not implement */
    LLAMA_ERR_WORKSPACE = -3,    /* workspace missing, too small or misaligned */
    LLAMA_ERR_HIP = -4,          /* the HIP runtime reported an error */
    LLAMA_STATUS_MAX_ENUM = 0x7FFFFFFF  /* not a status: makes every int32 a value of the type,
                                           so llama_status_str may be handed any code */
} llama_status;

typedef enum llama_dtype {
    LLAMA_BF16 = 0,  /* bf16 weights and KV cache; fp32 residual stream and accumulation */
    LLAMA_FP32 = 1,  /* fp32 weights, KV cache and arithmetic */
    LLAMA_FP16 = 2   /* fp16 weights and KV cache (the reference implementation's dtype): the
                        bf16 model's kernels in their fp16 form (MFMA prefill GEMMs and flash
                        attention, MFMA products for decode batches above 4, the vector GEMV
                        for batches of 1..4; GQA decode attention on the vector kernel), fp32
                        residual stream and accumulation, and the tensors the method stores in
                        16 bits (normalised operands, q, K/V, attention output, gated FFN
                        activation) rounded to fp16 (nearest even) where they are produced.
                        Weights 16-byte aligned, as for bf16 */
} llama_dtype;

/*
 * Structural configuration (Admin & Developer Guide, sections 3.3 and 8.4, ModelArgs).
 * head_dim = dim / n_heads; n_heads must be a multiple of n_kv_heads (grouped-query
 * attention: query head h reads kv head h / (n_heads / n_kv_heads), the repeat-interleave
 * of repeat_kv).  hidden_dim is the SwiGLU width, given explicitly (the multiple_of /
 * ffn_dim_multiplier rule of section 8.4 FeedForward is applied by the caller).
 * rope_theta is the RoPE base (10000 for Llama 2): pair i of a head at position t is
 * rotated by t * rope_theta^(-2i/head_dim), pairs being adjacent elements (2i, 2i+1).
 * max_batch_size and max_seq_len size the KV cache, which persists across calls
 * (section 6.2 "KV cache footprint").
 *
 * Supported: head_dim in {32, 64, 128}, n_heads / n_kv_heads in {1, 2, 4, 8}, even
 * vocab_size, dim, hidden_dim and
 * n_heads*head_dim multiples of 64, max_seq_len <= 65536.
 */
typedef struct llama_args {
    int32_t dim;
    int32_t n_layers;
    int32_t n_heads;
    int32_t n_kv_heads;
    int32_t vocab_size;
    int32_t hidden_dim;
    float norm_eps;
    float rope_theta;
    int32_t max_batch_size;
    int32_t max_seq_len;
    int32_t dtype;          /* llama_dtype */
} llama_args;

/*
 * Weights of one block, device pointers, element type = args.dtype, nn.Linear orientation
 * ([out_features][in_features], row-major, densely packed), bias-free (section 8.4):
 *   attention_norm, ffn_norm  [dim]
 *   wq  [n_heads*head_dim][dim]      row index = head*head_dim + d
 *   wk  [n_kv_heads*head_dim][dim]   row index = kv_head*head_dim + d
 *   wv  [n_kv_heads*head_dim][dim]
 *   wo  [dim][n_heads*head_dim]
 *   w1  [hidden_dim][dim]   (gate, passed through SiLU)
 *   w3  [hidden_dim][dim]   (up)
 *   w2  [dim][hidden_dim]   (down)
 * Every pointer must be 16-byte aligned.
 */
typedef struct llama_layer_weights {
    const void *attention_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w1, *w2, *w3;
} llama_layer_weights;

/*
 * tok_embeddings [vocab_size][dim], norm [dim], output [vocab_size][dim] (device), and
 * `layers`, a HOST array of n_layers llama_layer_weights, copied by llama_init.
 * Ownership: the weights are borrowed.  They stay owned by the caller, must remain valid
 * and unmodified until llama_destroy, and are never written by the library.
 */
typedef struct llama_weights {
    const void *tok_embeddings, *norm, *output;
    const llama_layer_weights *layers;
} llama_weights;

typedef struct llama_ctx llama_ctx;

/* Validates `a` on the host only (no device call).  LLAMA_OK, or the error llama_init
 * would return for these args. */
llama_status llama_check_args(const llama_args *a);

/* Bytes of device workspace llama_init needs for `a`: the KV cache
 * ([n_layers][max_batch_size][max_seq_len][n_kv_heads][head_dim], one array for K and one
 * for V, element type = dtype) plus activation scratch sized for a prefill of
 * max_batch_size * max_seq_len tokens.  Returns 0 if llama_check_args(a) != LLAMA_OK. */
size_t llama_workspace_bytes(const llama_args *a);

/* Creates a context.  d_workspace: device buffer of at least llama_workspace_bytes(a)
 * bytes, 256-byte aligned, owned by the caller, used exclusively by the ctx until
 * llama_destroy (the KV cache lives in it, so its contents persist between calls).
 * Uploads the RoPE cos/sin table (computed on the host in float64) on `stream`.
 * On success *out receives the ctx; on error *out is set to NULL. */
llama_status llama_init(const llama_args *a, const llama_weights *w, void *d_workspace,
                        size_t workspace_bytes, void *stream, llama_ctx **out);

/* Transformer.forward(tokens[:, 0:seqlen], start_pos) for batch rows [0, bsz):
 * d_tokens: int32 token ids, row b at d_tokens + b*ld_tokens, seqlen ids each (ld_tokens
 * >= seqlen).  Keys and values of positions [start_pos, start_pos+seqlen) are written to
 * the cache; attention reads cache positions [0, start_pos+seqlen) with the causal mask of
 * section 8.4 (query i sits at start_pos+i).  d_logits (fp32): all_positions == 0 ->
 * [bsz][vocab_size], logits of the last position of each row; all_positions != 0 ->
 * [bsz][seqlen][vocab_size].
 * Errors: INVALID_ARG if bsz < 1, bsz > max_batch_size, seqlen < 1, start_pos < 0,
 * start_pos + seqlen > max_seq_len, ld_tokens < seqlen, or a NULL pointer. */
llama_status llama_prefill(llama_ctx *c, const int32_t *d_tokens, int64_t ld_tokens,
                           int32_t bsz, int32_t seqlen, int32_t start_pos, float *d_logits,
                           int32_t all_positions, void *stream);

/* One single-token step, Transformer.forward(tokens[:, None], start_pos): row b's token is
 * d_tokens[b*ld_tokens].  Writes K/V at position start_pos, attends over
 * [0, start_pos] (no mask: every cached key is visible), and writes fp32 logits
 * [bsz][vocab_size] to d_logits.  Any bsz up to max_batch_size is served: 16-bit (bf16 or
 * fp16) batches of 5..32 rows stream the weights through the skinny MFMA kernels, larger
 * ones run the prefill GEMMs with the single-token attention kernel.
 * Errors: INVALID_ARG if bsz < 1, bsz > max_batch_size, start_pos < 0,
 * start_pos >= max_seq_len, ld_tokens < 1, or a NULL pointer. */
llama_status llama_decode_step(llama_ctx *c, const int32_t *d_tokens, int64_t ld_tokens,
                               int32_t bsz, int32_t start_pos, float *d_logits, void *stream);

/* llama_decode_step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation, the
 * same kernels and the same results, but the step's scratch (residual rows, q, the
 * projections' operands, attention split partials, K-split partials) lives in a static device
 * array of the library, 32 MiB, one per GPU, held until the process ends; the KV cache stays
 * in the ctx's workspace.  The call allocates nothing (no hipMalloc / hipFree, no graph, no
 * event; the HIP runtime loads the library's kernels at their first launch, so run one
 * ordinary call first where even that must not happen).  Every element of the array that a
 * call reads was written earlier in that call, so nothing in it needs clearing; the array
 * keeps the last call's contents.  All calls on one GPU share the array: calls that overlap
 * in time on one GPU (other streams, other threads, other ctxs) race and must be ordered by
 * the caller.
 * Errors: as llama_decode_step; UNSUPPORTED if bsz > 32; WORKSPACE if the step's scratch
 * exceeds the 32 MiB array (it needs about bsz * (3 * n_heads * head_dim + dim + hidden_dim)
 * * 4 bytes plus 64 * (dim + hidden_dim) bytes for 16-bit models and the attention partials);
 * HIP if the array's device address could not be taken at llama_init. */
llama_status llama_decode_step_noalloc(llama_ctx *c, const int32_t *d_tokens, int64_t ld_tokens,
                                       int32_t bsz, int32_t start_pos, float *d_logits, void *stream);

/* Greedy pick (section 8.5, temperature 0): d_out[b] = argmax_v d_logits[b*row_stride + v]
 * over v in [0, vocab); ties go to the lowest index; NaN entries are never picked (a row of
 * only NaN yields -1).  Independent of any ctx.
 * Errors: INVALID_ARG if bsz < 1, vocab < 1, row_stride < vocab or a NULL pointer. */
llama_status llama_argmax(const float *d_logits, int32_t bsz, int32_t vocab,
                          int64_t row_stride, int32_t *d_out, void *stream);

/* Temperature + top-p draw ([AG] section 8.5, temperature > 0: softmax(logits / temperature)
 * and then sample_top_p, which [ST] "Sampling, Stopping, and the Chat Template" describes as
 * sort descending, zero the tokens beyond the cumulative top-p mass, renormalise, draw one
 * token).  For each row b in [0, bsz), over v in [0, vocab):
 *   p = softmax(d_logits[b*row_stride + v] / temperature);
 *   tokens sorted by descending p, equal p by lower index;
 *   a token is dropped when the mass sorted before it exceeds top_p (the first token always
 *   stays; top_p >= 1 keeps every token); the kept mass is renormalised;
 *   d_out[b] = the first sorted kept token whose cumulative mass exceeds d_uniform[b]
 *   (a caller-supplied uniform in [0, 1); values outside are clamped into it).
 * If d_logprob is not NULL, d_logprob[b] = log_softmax(d_logits[b, :])[d_out[b]] (untempered).
 * Logits must be finite.  Buffers are device memory owned by the caller; d_out and d_logprob
 * are written only.  Sums are fp32 workgroup reductions: a uniform within ~1e-6 of a
 * cumulative boundary may select the neighbouring token relative to exact arithmetic.
 * Errors: INVALID_ARG if bsz < 1, vocab < 1, row_stride < vocab, temperature <= 0 or not
 * finite, top_p < 0 or NaN, or a NULL d_logits / d_uniform / d_out; UNSUPPORTED if
 * vocab > 32768. */
llama_status llama_sample_top_p(const float *d_logits, int32_t bsz, int32_t vocab, int64_t row_stride,
                                float temperature, float top_p, const float *d_uniform, int32_t *d_out,
                                float *d_logprob, void *stream);

/* Generate's token bookkeeping (section 8.5, torch.where on input_text_mask): for each row
 * b, if cur_pos >= d_prompt_len[b] then d_tokens[b*ld_tokens + cur_pos] = d_next[b];
 * otherwise the prompt token already there is kept.
 * Errors: INVALID_ARG if bsz < 1, cur_pos < 0, cur_pos >= ld_tokens or a NULL pointer. */
llama_status llama_select_next(const int32_t *d_next, int32_t *d_tokens, int64_t ld_tokens,
                               int32_t cur_pos, const int32_t *d_prompt_len, int32_t bsz,
                               void *stream);

/*
 * Diagnostics: device time of one class of kernel launches.  llama_profile_select(c, k)
 * makes the ctx time every kernel it later launches for class k (LLAMA_KC_*, 0 = none):
 * each such kernel is dispatched with hipExtLaunchKernel and an event pair that HIP binds
 * to that dispatch's own begin and end.  llama_profile_read waits for those events, returns
 * the number of timed kernels and their summed duration in milliseconds, and forgets them.
 * The calling thread is the one whose launches are timed.  Meant for measurement runs: the
 * timed dispatches carry profiling timestamps.
 * Errors: INVALID_ARG for a NULL ctx/pointer or an unknown class; HIP on event failure.
 */
enum llama_kernel_class {
    LLAMA_KC_NONE = 0,
    LLAMA_KC_GEMV_QKV = 1,    /* decode: fused RMSNorm + [wq;wk;wv] + RoPE + KV append */
    LLAMA_KC_ATTN_DECODE = 2, /* decode: split attention (+ merge) */
    LLAMA_KC_GEMV_WO = 3,     /* decode: wo + residual */
    LLAMA_KC_GEMV_W13 = 4,    /* decode: fused RMSNorm + [w1;w3] + SiLU gate */
    LLAMA_KC_GEMV_W2 = 5,     /* decode: w2 + residual */
    LLAMA_KC_GEMV_OUT = 6,    /* final RMSNorm + vocab projection (decode and prefill) */
    LLAMA_KC_GEMM_QKV = 7,    /* prefill: MFMA [wq;wk;wv] + RoPE + KV append */
    LLAMA_KC_ATTN_PREFILL = 8,/* prefill: causal attention */
    LLAMA_KC_GEMM_WO = 9,     /* prefill: MFMA wo + residual */
    LLAMA_KC_GEMM_W13 = 10,   /* prefill: MFMA [w1;w3] + SiLU gate */
    LLAMA_KC_GEMM_W2 = 11,    /* prefill: MFMA w2 + residual */
    LLAMA_KC_RMSNORM = 12,    /* prefill: RMSNorm to the 16-bit storage type */
    LLAMA_KC_COUNT = 13
};
llama_status llama_profile_select(llama_ctx *c, int32_t kernel_class);
llama_status llama_profile_read(llama_ctx *c, int64_t *launches, double *total_ms);

/* Releases the ctx (host memory only; the workspace and weights stay the caller's).
 * Waits for nothing: the caller must not destroy a ctx with work still in flight. */
void llama_destroy(llama_ctx *c);

/* Static, human-readable name of a status code. */
const char *llama_status_str(llama_status st);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_MI355X_H */
