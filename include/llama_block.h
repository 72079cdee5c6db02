/*
 * llama_block.h - C ABI of the MI355X (gfx950) LLaMA decoder-block forward pass.
 *
 * The block is the pre-norm decoder layer of the consolidated single-GPU LLaMA
 * code ("LLaMA: Open and Efficient Foundation Language Models" notes, section 3
 * "代码实现": ModelArgs, RMSNorm, precompute_freqs_cis, apply_rotary_emb,
 * repeat_kv, Attention, FeedForward, TransformerBlock):
 *
 *     h   = x + wo( GQA-attention( RoPE(wq xn), RoPE(wk xn), wv xn ) ),  xn = RMSNorm(x)
 *     out = h + w2( silu(w1 hn) * (w3 hn) ),                             hn = RMSNorm(h)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers marked "device" point to GPU memory owned by the caller; the
 *    library allocates nothing, keeps no pointer after returning and has no
 *    mutable global state (calls on different streams may run concurrently as
 *    long as they do not write the same buffers).
 *  - All tensors are dense and row-major.  Activations are [rows, features];
 *    linear weights are stored as nn.Linear stores them, [out_features,
 *    in_features], and applied as y = x W^T; the KV cache is
 *    [max_batch_size, max_seq_len, n_kv_heads, head_dim].
 *  - Element type: LLAMA_BF16 (bfloat16 storage, fp32 arithmetic inside, one
 *    round-to-nearest-even rounding per stored value) or LLAMA_F32.  Every
 *    tensor of a call has the call's dtype unless stated otherwise (the RoPE
 *    table and LM-head logits are always fp32, token ids int32).
 *  - Device pointers must be 16-byte aligned (tensors are moved in 16-byte
 *    vectors and global -> LDS copies), except int32 arrays (token ids, chosen
 *    ids, the device-resident position) and the per-row uniforms of
 *    llama_sample_top_p, which need 4-byte alignment.  A misaligned pointer is
 *    rejected with LLAMA_ERR_INVALID_ARG.
 *  - Device entry points only enqueue work on `stream` (a hipStream_t; NULL is
 *    the default stream) and return without synchronising.  Results are ready
 *    when the stream reaches that point.
 *  - Every argument is validated on the host before anything is enqueued: on a
 *    non-zero return nothing was launched and no buffer was touched.
 *  - No exception crosses the ABI and nothing aborts.
 */
#ifndef LLAMA_BLOCK_H
#define LLAMA_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* llama_stream_t; /* the same type as hipStream_t */

/* Return codes. */
enum {
  LLAMA_OK = 0,
  LLAMA_ERR_INVALID_ARG = -1,        /* null pointer, bad size or inconsistent shape */
  LLAMA_ERR_UNSUPPORTED = -2,        /* valid but not built: dtype/head_dim combination */
  LLAMA_ERR_WORKSPACE_TOO_SMALL = -3,/* ws_bytes below the size the *_workspace_size call reports */
  LLAMA_ERR_HIP = -4,                /* a HIP launch reported an error */
  LLAMA_ERR_SCRATCH_TOO_SMALL = -5   /* an allocation-free call needs more than its static scratch */
};

typedef enum { LLAMA_F32 = 0, LLAMA_BF16 = 1 } llama_dtype;

/*
 * Model hyper-parameters: the ModelArgs dataclass of the notes' section 3,
 * plus rope_theta from "灵哥讲llama3(中)" (Transformer.__init__ passes
 * params.rope_theta to precompute_freqs_cis).
 *   n_kv_heads  <= 0 means "None", i.e. equal to n_heads.
 *   ffn_dim_multiplier <= 0 means "None".
 *   head_dim = dim / n_heads; n_rep = n_heads / n_kv_heads.
 */
typedef struct {
  int32_t dim;
  int32_t n_layers;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t vocab_size;
  int32_t multiple_of;
  float ffn_dim_multiplier;
  float norm_eps;
  float rope_theta;
  int32_t max_batch_size;
  int32_t max_seq_len;
} llama_model_args;

/* The nine parameter tensors of one TransformerBlock (device pointers):
 * attention_norm, ffn_norm [dim]; wq [n_heads*head_dim, dim];
 * wk, wv [n_kv_heads*head_dim, dim]; wo [dim, n_heads*head_dim];
 * w1, w3 [hidden, dim]; w2 [dim, hidden]. */
typedef struct {
  const void* attention_norm;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const void* ffn_norm;
  const void* w1;
  const void* w2;
  const void* w3;
} llama_block_weights;

/* ------------------------------------------------------------------ host-only helpers */

/* Text for a return code.  Never NULL. */
const char* llama_status_str(int status);

/* FeedForward width (notes, section 3, FeedForward.__init__ with hidden = 4*dim):
 * int(2*hidden/3), times ffn_dim_multiplier truncated to int when set, rounded up
 * to a multiple of multiple_of.  Writes *hidden.  Host only. */
int llama_ffn_hidden_dim(const llama_model_args* args, int32_t* hidden);

/* Workspace bytes llama_block_forward needs for a call of bsz x seqlen tokens
 * at start_pos (decode partials depend on the attended length).  Host only. */
int llama_block_workspace_size(const llama_model_args* args, int32_t bsz, int32_t seqlen,
                               int32_t start_pos, llama_dtype dtype, size_t* bytes);

/* Workspace bytes llama_gqa_attn_decode needs (split-K partial results). Host only. */
int llama_attn_decode_workspace_size(const llama_model_args* args, int32_t bsz, int32_t start_pos,
                                     size_t* bytes);

/* Workspace bytes llama_swiglu_ffn needs for `rows` rows of width `dim` (the gated
 * [rows, hidden] activation plus split-K partial sums for small row counts).  Host only. */
int llama_ffn_workspace_size(int64_t rows, int32_t dim, int32_t hidden, llama_dtype dtype, size_t* bytes);

/* ------------------------------------------------------------------ device entry points */

/* RoPE table (notes, section 3, precompute_freqs_cis): for p < end and
 * i < head_dim/2, freqs_cis[p][i] = (cos(p*t_i), sin(p*t_i)) with
 * t_i = rope_theta^(-2i/head_dim).  Angles and cos/sin are evaluated in fp64 on
 * the device and stored as fp32 pairs: freqs_cis is device float[end][head_dim/2][2].
 * Requires head_dim even, end >= 1. */
int llama_rope_freqs(float* freqs_cis, int32_t head_dim, int32_t end, float rope_theta,
                     llama_stream_t stream);

/* RMSNorm (notes, section 3, class RMSNorm): y[r][c] = x[r][c] / sqrt(mean_c x[r][c]^2 + eps) * w[c].
 * x, y: device [rows][dim]; w: device [dim].  Sum of squares in fp32.  y may equal x
 * (in place).  Requires rows >= 0 (0 is a no-op), dim >= 1, dim % 8 == 0 for
 * bf16 and dim % 4 == 0 for f32. */
int llama_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int32_t dim, float eps,
                  llama_dtype dtype, llama_stream_t stream);

/* RoPE in place (notes, section 3, apply_rotary_emb): every head vector u of xq
 * [bsz][seqlen][n_heads][head_dim] and xk [bsz][seqlen][n_kv_heads][head_dim] at
 * sequence index s has each interleaved pair (u[2i], u[2i+1]) rotated by the angle of
 * freqs_cis[start_pos + s][i] (a llama_rope_freqs table with freqs_end rows).
 * xk may be NULL (only q rotated).  Requires head_dim a multiple of 4 (two
 * pairs per vector), start_pos + seqlen <= freqs_end. */
int llama_rope(void* xq, void* xk, const float* freqs_cis, int32_t freqs_end, int32_t bsz,
               int32_t seqlen, int32_t start_pos, int32_t n_heads, int32_t n_kv_heads,
               int32_t head_dim, llama_dtype dtype, llama_stream_t stream);

/* Prefill attention with cache append (notes, section 3, Attention.forward from the
 * cache write to the head concatenation; causal mask with cache offset from
 * "灵哥讲llama3(中)", Transformer forward):
 *   cache_k[b][start_pos+s] = xk[b][s], cache_v[b][start_pos+s] = xv[b][s]   (s < seqlen)
 *   out[b][s][h*d:(h+1)*d] = sum_{t <= start_pos+s} softmax_t(q.k_t/sqrt(d)) v_t,
 *   with q = xq[b][s][h] and the kv head h / n_rep.
 * xq: device [bsz][seqlen][n_heads][d] (already rotated); xk, xv: device
 * [bsz][seqlen][n_kv_heads][d] (xk already rotated); cache_k, cache_v: device
 * [max_batch_size][max_seq_len][n_kv_heads][d]; out: device [bsz][seqlen][n_heads*d].
 * Only cache rows [:bsz][start_pos:start_pos+seqlen] are written.
 * Requires 1 <= bsz <= max_batch_size, seqlen >= 1, start_pos >= 0,
 * start_pos + seqlen <= max_seq_len, n_heads % n_kv_heads == 0,
 * head_dim in {32, 64, 128} (bf16: {64, 128}). */
int llama_gqa_attn_prefill(const void* xq, const void* xk, const void* xv, void* cache_k,
                           void* cache_v, void* out, const llama_model_args* args, int32_t bsz,
                           int32_t seqlen, int32_t start_pos, llama_dtype dtype,
                           llama_stream_t stream);

/* Single-token decode attention (seqlen = 1, no mask: every cached position up to and
 * including start_pos is visible).  Same layouts as the prefill call with seqlen = 1;
 * appends xk, xv at start_pos, then attends over start_pos + 1 keys with a split-K
 * pass whose fp32 partials go to `ws` (device, ws_bytes >=
 * llama_attn_decode_workspace_size).  Requires start_pos + 1 <= max_seq_len. */
int llama_gqa_attn_decode(const void* xq, const void* xk, const void* xv, void* cache_k,
                          void* cache_v, void* out, const llama_model_args* args, int32_t bsz,
                          int32_t start_pos, void* ws, size_t ws_bytes, llama_dtype dtype,
                          llama_stream_t stream);

/* Allocation-free variant of llama_gqa_attn_decode, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, kernels and results,
 * with the split-K partials in a static device array of the library instead of
 * a caller workspace.  Each GPU holds its own copy of the array (8 MiB, see
 * llama_static_scratch_bytes) from the first call on that device until the
 * process ends; the call makes no hipMalloc/hipFree and allocates nothing else.
 * Call it with the device of `stream` current (its scratch address is looked up
 * for the current device).  A call whose partials
 * (bsz * n_heads * splits * (head_dim + 2) floats, the same count as
 * llama_attn_decode_workspace_size reports) exceed the array returns
 * LLAMA_ERR_SCRATCH_TOO_SMALL before anything is enqueued.  Every call on one
 * GPU shares that GPU's array and nothing in it needs clearing between calls;
 * calls that can overlap on one GPU (different streams) race on it and must be
 * ordered by the caller.  Arguments, layouts and other errors as
 * llama_gqa_attn_decode. */
int llama_gqa_attn_decode_static(const void* xq, const void* xk, const void* xv, void* cache_k,
                                 void* cache_v, void* out, const llama_model_args* args,
                                 int32_t bsz, int32_t start_pos, llama_dtype dtype,
                                 llama_stream_t stream);

/* Size in bytes of the static scratch array behind llama_gqa_attn_decode_static.  Host only. */
size_t llama_static_scratch_bytes(void);

/* SwiGLU feed-forward without residual (notes, section 3, FeedForward.forward):
 * y = w2( silu(w1 x) * (w3 x) ), silu(a) = a / (1 + e^-a).
 * x: device [rows][dim]; w1, w3: device [hidden][dim]; w2: device [dim][hidden];
 * y: device [rows][dim]; ws: device, ws_bytes >= llama_ffn_workspace_size.
 * Requires dim % 8 == 0 and hidden % 8 == 0 for bf16 (dim, hidden % 4 == 0 for f32). */
int llama_swiglu_ffn(const void* x, const void* w1, const void* w3, const void* w2, void* y,
                     int64_t rows, int32_t dim, int32_t hidden, void* ws, size_t ws_bytes,
                     llama_dtype dtype, llama_stream_t stream);

/* Plain projection y = x W^T (nn.Linear without bias).  x: device [rows][in];
 * w: device [out][in]; y: device [rows][out].  Requires in % 8 == 0 and
 * out % 4 == 0 for bf16 (in, out % 4 == 0 for f32).  Takes no workspace, so K
 * is never split: for 5..64 rows and few output columns the grid is small
 * (the block calls split those projections through their workspace). */
int llama_linear(const void* x, const void* w, void* y, int64_t rows, int32_t in_features,
                 int32_t out_features, llama_dtype dtype, llama_stream_t stream);

/* One decoder block (notes, section 3, TransformerBlock.forward):
 *   h = x + Attention(RMSNorm(x)); out = h + FeedForward(RMSNorm(h)).
 * x, out: device [bsz][seqlen][dim], out must not overlap x; cache_k/cache_v as in
 * llama_gqa_attn_prefill (rows [:bsz][start_pos:start_pos+seqlen] written with k
 * after RoPE and v); freqs_cis: llama_rope_freqs table with freqs_end rows, head_dim
 * = dim / n_heads.  seqlen == 1 takes the decode path (split-K attention), seqlen > 1
 * the prefill path (causal mask with cache offset).  ws: device, ws_bytes >=
 * llama_block_workspace_size(args, bsz, seqlen, start_pos, dtype).
 * Requires everything llama_gqa_attn_prefill requires, start_pos + seqlen <= freqs_end,
 * dim % 8 == 0 and hidden % 8 == 0 for bf16 (% 4 for f32). */
int llama_block_forward(const llama_model_args* args, const llama_block_weights* weights,
                        void* cache_k, void* cache_v, const float* freqs_cis, int32_t freqs_end,
                        const void* x, void* out, int32_t bsz, int32_t seqlen, int32_t start_pos,
                        void* ws, size_t ws_bytes, llama_dtype dtype, llama_stream_t stream);

/* llama_block_forward with stage timing: identical arguments and results, plus
 * `events`, 8 caller-created hipEvent_t handles recorded on `stream`: events[0]
 * before the first kernel and events[i] after stage i, the stages being
 * 1 attention_norm, 2 QKV projection + RoPE + cache append, 3 attention,
 * 4 wo + residual, 5 ffn_norm, 6 w1/w3 + SwiGLU, 7 w2 + residual.
 * hipEventElapsedTime(events[i-1], events[i]) is stage i's duration.  Calls of
 * one to four tokens normalise inside stages 2 and 6, and bf16 calls of 5 to 64
 * tokens whose wo projection is split over K compute ffn_norm inside stage 4:
 * the normalisation stages then hold no kernel. */
int llama_block_forward_events(const llama_model_args* args, const llama_block_weights* weights,
                               void* cache_k, void* cache_v, const float* freqs_cis,
                               int32_t freqs_end, const void* x, void* out, int32_t bsz,
                               int32_t seqlen, int32_t start_pos, void* ws, size_t ws_bytes,
                               llama_dtype dtype, llama_stream_t stream, void* const* events);

/* One-token decode of the block at a position held in device memory (the
 * generate loop of the linkmax.top walkthrough, section 3.3, feeds each new
 * token back at start_pos + 1): identical to llama_block_forward with
 * seqlen = 1 and start_pos = *start_pos_dev, except that the position is read
 * by the kernels when they execute, so one recorded call (e.g. in a captured
 * HIP graph) can be replayed at successive positions by advancing
 * *start_pos_dev on the device between replays.
 *   start_pos_dev: device int32, 4-byte aligned, shared by all bsz rows.
 *   max_start_pos: the largest position the call may see.  The host validates
 *     max_start_pos + 1 <= max_seq_len and <= freqs_end, and sizes the
 *     workspace and the attention splits for it: ws_bytes >=
 *     llama_block_workspace_size(args, bsz, 1, max_start_pos, dtype).
 *   The caller guarantees 0 <= *start_pos_dev <= max_start_pos when the call
 *   runs; the kernels clamp the value into that range (so memory accesses stay
 *   inside the caches) but cannot report a violation.
 * bf16 only (LLAMA_ERR_UNSUPPORTED for fp32); other arguments and errors as
 * llama_block_forward. */
int llama_block_decode_at(const llama_model_args* args, const llama_block_weights* weights,
                          void* cache_k, void* cache_v, const float* freqs_cis, int32_t freqs_end,
                          const void* x, void* out, int32_t bsz, const int32_t* start_pos_dev,
                          int32_t max_start_pos, void* ws, size_t ws_bytes, llama_dtype dtype,
                          llama_stream_t stream);

/* Token embedding lookup (notes, section 3, Transformer.forward, tok_embeddings):
 * out[i] = table[tokens[i]].  tokens: device int32 [n]; table: device [vocab][dim];
 * out: device [n][dim].  Ids outside [0, vocab) produce a zero row (checked on the
 * device; the host cannot see the ids). */
int llama_embedding(const int32_t* tokens, const void* table, void* out, int64_t n, int32_t dim,
                    int32_t vocab, llama_dtype dtype, llama_stream_t stream);

/* Final RMSNorm + output projection of one row per sequence + greedy token
 * (linkmax.top walkthrough, section 3.2.2 Transformer.forward on h[:, -1], and
 * section 3.3 generate, argmax when temperature is 0; lowest id wins exact ties):
 *   logits[b] = RMSNorm(h[b], norm_w, eps) W_out^T  (fp32),  next[b] = argmax logits[b].
 * h: device [bsz] rows of dim elements, row b at h + b*h_row_stride elements;
 * norm_w: device [dim]; w_out: device [vocab][dim]; logits: device float [bsz][vocab];
 * next: device int32 [bsz]; ws: device, ws_bytes >= llama_lm_head_workspace_size. */
int llama_lm_head_workspace_size(int32_t bsz, int32_t dim, int32_t vocab, llama_dtype dtype,
                                 size_t* bytes);
int llama_lm_head_argmax(const void* h, int64_t h_row_stride, const void* norm_w,
                         const void* w_out, float* logits, int32_t* next, int32_t bsz,
                         int32_t dim, int32_t vocab, float eps, void* ws, size_t ws_bytes,
                         llama_dtype dtype, llama_stream_t stream);

/* Next token per row by temperature + nucleus (top-p) sampling (linkmax.top walkthrough,
 * section 3.3, generate and sample_top_p): probabilities softmax(logits / temperature);
 * tokens in descending probability, equal probabilities by ascending id; a token is kept
 * when the probability before it in that order is <= top_p (the first is always kept);
 * the kept probabilities are renormalised and the token drawn is the first whose
 * cumulative kept probability exceeds uniforms[b] (inverse-CDF draw: uniforms[b] in
 * [0, 1) supplies the randomness, so the call is deterministic).  temperature <= 0 takes
 * the argmax (lowest id among equal maxima) and ignores top_p and uniforms.
 * logits: device float [bsz][vocab], finite; next: device int32 [bsz]; uniforms: device
 * float [bsz] (may be NULL when temperature <= 0).  Requires top_p not NaN.  No workspace;
 * the arithmetic is fp32 per token with fp64 sums, deterministic for given inputs. */
int llama_sample_top_p(const float* logits, int32_t* next, int32_t bsz, int32_t vocab,
                       float temperature, float top_p, const float* uniforms,
                       llama_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_BLOCK_H */
