/* gptmi.h -- C ABI of the MI355X (gfx950) GPT-2-style decoder-only forward pass.
 *
 * The model (pages cited by title and section):
 *   x = E[idx] + P[t]                                   "第 25 章 从小 GPT 到 GPT-2" §25.1
 *   per block (pre-norm):                               §25.1; "预训练一个 Mini GPT" 第4步
 *     a = LN1(x);  qkv = a W_attn^T + b_attn            §25.2 (fused c_attn, split Q|K|U)
 *     per head: Y = softmax(Q K^T / sqrt(D) + M) U       §25.2 (M = -inf where s > t)
 *     x += concat_h(Y) W_proj^T + b_proj                 §25.2 (c_proj)
 *     x += gelu_tanh(LN2(x) W_fc^T + b_fc) W_fp^T + b_fp §25.3; "GPT-1学习笔记" §3.6
 *   logits = LN_f(x) E^T   (tied head, same E)          §25.4
 *   loss   = mean over predicted positions of logsumexp(z) - z[y]
 *                                                       "预训练一个 Mini GPT" 第6步; §25.7
 *   LayerNorm: biased variance, eps inside the square root ("GPT-1学习笔记" §3.2).
 *
 * Conventions for every entry point:
 *  - Buffers marked (device) are device pointers owned by the caller; (host)
 *    are host pointers.  The library never allocates, never frees, keeps no
 *    state between calls (gpt_decode_step_noalloc's static device array
 *    aside), never synchronises and enqueues work only on `stream` (a
 *    hipStream_t; NULL = the default stream).
 *  - Every host-checkable condition is checked before the first HIP call; on
 *    an error nothing is enqueued and the outputs are untouched.  A HIP
 *    launch failure returns GPT_ERR_HIP (the HIP code is not kept); outputs
 *    are then undefined.
 *  - Device buffers must be 16-byte aligned (every HIP or torch allocation
 *    is); the parameter blob's tensors then are too, since every tensor
 *    size is a multiple of C or n_ff.
 *  - Matrices are row-major [out, in]; a linear layer is y = x W^T + b.
 *  - dtype GPT_F32: parameters, activations and outputs fp32, MFMA in fp32.
 *    dtype GPT_BF16: parameters, activations and logits bf16 (round to
 *    nearest even), fp32 accumulation, fp32 residual stream, fp32 losses.
 *  - Token ids outside [0, V) violate the contract: the kernels clamp them
 *    to stay in bounds, and the results are then unspecified.
 */
#ifndef GPTMI_H
#define GPTMI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gpt_dtype { GPT_F32 = 0, GPT_BF16 = 1 };

enum gpt_status {
  GPT_OK = 0,
  GPT_ERR_NULL = -1,          /* a required pointer is NULL */
  GPT_ERR_CONFIG = -2,        /* dims <= 0, C % H != 0, C % 8 != 0, n_ff % 8 != 0, D % 8 != 0 or D > 128 */
  GPT_ERR_SEQ_TOO_LONG = -3,  /* T > ctx ("Day 16 从零组装 MiniGPT" 三十九: longer inputs are rejected) */
  GPT_ERR_SHAPE = -4,         /* B <= 0, T <= 0, or a shape argument out of range */
  GPT_ERR_WORKSPACE = -5,     /* ws_bytes smaller than gpt_workspace_bytes() */
  GPT_ERR_DTYPE = -6,         /* dtype not GPT_F32 / GPT_BF16 */
  GPT_ERR_HIP = -7            /* a kernel launch failed */
};

/* Model configuration (host).  n_ff is the MLP width (4 * n_embd for GPT-2,
 * "第 25 章 从小 GPT 到 GPT-2" §25.3).  ln_eps is 1e-5 for every model here.
 * The last three fields select the variants the pages describe besides GPT-2
 * (all 0 for GPT-2):
 *   activation   0: tanh GELU ("GPT-1学习笔记" §3.6 approximation; §25.3);
 *                1: exact GELU 0.5 z (1 + erf(z / sqrt 2)) ("GPT-1学习笔记"
 *                §3.6 standard formula; "Day 16" nn.GELU()).
 *   post_ln      0: pre-LN blocks and a final LayerNorm (GPT-2);
 *                1: post-LN blocks, n = LN1(x + attn(x)), h = LN2(n + mlp(n)),
 *                and no final LayerNorm ("GPT-1学习笔记" §3.1-§3.2, §4.1).
 *   untied_head  0: the head reuses the token table (tying);
 *                1: a separate head matrix [V, C] without bias ("Day 16" 二十三). */
typedef struct gpt_config {
  int32_t vocab;    /* V */
  int32_t ctx;      /* maximum sequence length (rows of the position table) */
  int32_t n_embd;   /* C */
  int32_t n_head;   /* H; head width D = C / H */
  int32_t n_layer;  /* L */
  int32_t n_ff;     /* MLP hidden width */
  float ln_eps;
  int32_t dtype;    /* enum gpt_dtype */
  int32_t activation;
  int32_t post_ln;
  int32_t untied_head;
  int32_t arch;       /* 0: GPT-2 blocks; 1: LLaMA-style blocks ("02 GPT 架构" §6.1-6.3):
                       * RMSNorm g*x/sqrt(mean(x^2)+ln_eps) in place of LayerNorm, no position
                       * table, RoPE on Q and K (adjacent pairs (2i, 2i+1) turned by
                       * p * rope_theta^(-2i/D), §5.2), grouped-query attention (§6.2),
                       * SwiGLU MLP W2(SiLU(x W1) * (x W3)), no biases, a final RMSNorm.
                       * activation and post_ln must be 0. */
  int32_t n_kv_head;  /* arch 1: K/V heads (divides n_head; 1 = MQA; 0 = n_head).  arch 0: 0 or n_head. */
  float rope_theta;   /* arch 1: RoPE base (the pages use 10000); > 0 */
  int32_t alibi;      /* arch 1 only: 1 = ALiBi in place of RoPE ("02 GPT 架构" §5.3): the scores
                       * carry -m_h |i - j|, m_h = 2^(-8 (h+1) / H) (no rotation); 0 otherwise */
} gpt_config;

/* Number of unique parameters, closed form ("第 25 章 从小 GPT 到 GPT-2" §25.4):
 * L(4C^2+4C + 2C*F+F+C + 4C) + VC + ctx*C + 2C, which is L(12C^2+13C)+VC+ctx*C+2C
 * at F = 4C; a post-LN model has no final LayerNorm (no 2C), an untied head
 * adds VC.  Also the element count of the parameter blob.  Returns a
 * negative gpt_status on an invalid config (host only, no HIP call). */
int64_t gpt_param_count(const gpt_config* cfg);
/*   (arch 1: per block 2C + (C + 2 Hkv D) C + C^2 + 3 C F, plus VC, the final
 *   RMSNorm's C and, untied, VC.) */

/* Element offsets of every tensor in the parameter blob, in packing order:
 *   wte[V,C], wpe[ctx,C],
 *   per layer l: ln1_g[C], ln1_b[C], attn_w[3C,C], attn_b[3C], proj_w[C,C], proj_b[C],
 *                ln2_g[C], ln2_b[C], fc_w[F,C], fc_b[F], fcproj_w[C,F], fcproj_b[C],
 *   lnf_g[C], lnf_b[C]   (pre-LN models only),
 *   head_w[V,C]          (untied head only),
 *   end.
 * arch 1 (LLaMA-style):
 *   wte[V,C],
 *   per layer l: rms1_g[C], wqkv[(H + 2 Hkv) D, C] (rows of W_q, then W_k, W_v),
 *                wo[C,C], rms2_g[C], w13[2F, C] (rows interleaved: 2j = gate W1
 *                row j, 2j+1 = up W3 row j), w2[C,F],
 *   rmsf_g[C], head_w[V,C] (untied head only), end: 1 + 6 L + 1 (+1) + 1 offsets.
 * With a tied head there is no head tensor: the head reads wte (tying as one
 * shared tensor, §25.4).  off (host) receives 2 + 12 L + (post_ln ? 0 : 2) +
 * (untied_head ? 1 : 0) + 1 values.  Returns GPT_OK, or GPT_ERR_SHAPE if n is
 * too small (host only). */
int gpt_param_offsets(const gpt_config* cfg, int64_t* off, int n);

/* Device workspace bytes needed by gpt_forward for a [B, T] batch (host only). */
int gpt_workspace_bytes(const gpt_config* cfg, int B, int T, size_t* bytes);

/* Forward pass + next-token cross-entropy.
 *   params     (device) blob of gpt_param_count() elements in cfg->dtype.
 *   idx        (device) int32 [B, T] token ids in [0, V).
 *   targets    (device, nullable) int32 [B, T]; -1 = no target.  NULL means
 *              derived targets y[b,t] = idx[b,t+1] for t < T-1 and none at the
 *              last position (§25.7: shift once).
 *   logits     (device, nullable) [B, T, V] in cfg->dtype; NULL skips writing
 *              them (the loss is still computed, from fp32 accumulators).
 *   token_loss (device, nullable) fp32 [B, T]; 0 where there is no target.
 *   mean_loss  (device, nullable) fp32 [1]; mean over positions with a
 *              target (NaN if there are none).
 *   ws         (device) workspace of at least gpt_workspace_bytes(cfg,B,T).
 * Requires 1 <= T <= ctx. */
int gpt_forward(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                const int32_t* targets, void* logits, float* token_loss, float* mean_loss,
                void* ws, size_t ws_bytes, void* stream);

/* gpt_forward with the logits rows ld_logits elements apart: logits is
 * [B, T, ld_logits] with ld_logits >= V, columns V .. ld_logits - 1 of every
 * row left untouched (ld_logits = V, or 0, is gpt_forward).  In bf16, a
 * stride that is a multiple of 64 elements with a 128-byte aligned base puts
 * every row on 128-byte lines; the head then writes whole lines and keeps
 * them out of the L2 cache (for GPT-2, ld_logits = 50304: the logits then
 * cost less time than dense rows of 50257).  Errors as gpt_forward, and
 * GPT_ERR_SHAPE for ld_logits < V or > 2^31. */
int gpt_forward_ld(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                   const int32_t* targets, void* logits, long long ld_logits, float* token_loss, float* mean_loss,
                   void* ws, size_t ws_bytes, void* stream);

/* Kernel classes for gpt_forward_timed. */
enum gpt_kernel {
  GPT_KERNEL_HEAD = 0,   /* tied head GEMM + cross-entropy partials (one launch per forward) */
  GPT_KERNEL_QKV = 1,    /* c_attn GEMM + Q/K/U scatter (last layer's launch) */
  GPT_KERNEL_ATTN = 2,   /* flash attention (last layer's launch) */
  GPT_KERNEL_PROJ = 3,   /* c_proj GEMM + residual (last layer's launch) */
  GPT_KERNEL_FC = 4,     /* c_fc GEMM + GELU (last layer's launch) */
  GPT_KERNEL_FCPROJ = 5, /* mlp.c_proj GEMM + residual (last layer's launch) */
  GPT_KERNEL_LN = 6      /* ln_2 LayerNorm (last layer's launch) */
};

/* gpt_forward_ld with a timing hook: ev_begin and ev_end (hipEvent_t,
 * created by the caller, nullable) are recorded on `stream` immediately
 * before and after the launch of kernel class `which`.  Everything else is
 * gpt_forward_ld. */
int gpt_forward_timed(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                      const int32_t* targets, void* logits, long long ld_logits, float* token_loss,
                      float* mean_loss, void* ws, size_t ws_bytes, void* stream, void* ev_begin, void* ev_end,
                      int which);

/* ---- greedy decoding with a key/value cache ----
 * "预训练一个 Mini GPT" (KV cache section, 第7步): a new token computes only
 * its own q, k and u; the keys and values of earlier positions are read back
 * from a per-layer cache.  "GPT-1学习笔记" §6.1: the next token is the argmax of
 * the last position's logits (lowest index on ties).
 *
 * Cache layout (device, caller-owned, cfg->dtype): k_cache and v_cache each
 * [L][B][Hkv][Tmax][D] (Hkv = K/V heads: n_head for GPT-2 blocks); row t of
 * (l, b, h) holds position t (arch 1: the key after its rotation).  Requires
 * 1 <= Tmax <= min(ctx, 4096).  pos (device, int32[1]) is the number of cache
 * positions already filled, the same for every sequence; the library updates
 * it on the device, so a decode loop needs no host round trip.
 * A position outside [0, Tmax) at a step violates the contract: nothing is
 * written outside the caches and the results are unspecified. */

/* Workspace bytes for gpt_prefill on a [B, Tp] prompt batch; it also covers
 * gpt_decode_step at the same B (host only). */
int gpt_decode_workspace_bytes(const gpt_config* cfg, int B, int Tp, size_t* bytes);

/* Prefill: the forward pass over prompts idx (device, int32 [B, Tp]) at
 * positions 0..Tp-1, storing every layer's K and U in the caches, then ln_f
 * and the tied head on the last position of each sequence only.
 *   next_tok    (device) int32 [B]: argmax of the last position's logits.
 *   last_logits (device, nullable) [B, V] in cfg->dtype.
 *   pos         (device) int32[1]: set to Tp.
 * Requires 1 <= Tp <= Tmax; else GPT_ERR_SEQ_TOO_LONG. */
int gpt_prefill(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int Tp,
                void* k_cache, void* v_cache, int Tmax, int32_t* pos, int32_t* next_tok,
                void* last_logits, void* ws, size_t ws_bytes, void* stream);

/* One decode step: tok (device, int32 [B]) enters at position p = *pos; its
 * K and U are appended at row p of every layer's cache and its query attends
 * over rows 0..p.  Writes next_tok (device, int32 [B]; may alias tok) and,
 * if logits (device, [B, V], cfg->dtype) is not NULL, the step's logits; then
 * *pos = p + 1.  ws as for gpt_prefill at this B (or larger). */
int gpt_decode_step(const gpt_config* cfg, const void* params, const int32_t* tok, int B, int32_t* pos,
                    void* k_cache, void* v_cache, int Tmax, int32_t* next_tok, void* logits,
                    void* ws, size_t ws_bytes, void* stream);

/* ---- a decode step that allocates nothing ----
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Exactly gpt_decode_step (same arguments, results and errors),
 * except that the workspace is a library-owned static device array of
 * GPT_DECODE_NOALLOC_BYTES (8 MiB) per GPU, allocated when the library is
 * loaded and held until the process ends; its device address is looked up
 * (hipGetSymbolAddress) on the first call on each device.  The call itself
 * allocates and frees nothing.
 *   Limit: the step's workspace at this B must fit, or GPT_ERR_WORKSPACE
 *   (GPT-2 124M in bf16 fits up to B = 64: 5.3 MB).
 *   Sharing: every call on one GPU uses that GPU's single array, which keeps
 *   the previous call's contents (the step clears what must start at zero
 *   itself); calls that overlap on one GPU (other streams or threads) race
 *   on it, so the caller serialises them.
 *   Errors: as gpt_decode_step; GPT_ERR_HIP if the array's address cannot be
 *   obtained on the current device. */
#define GPT_DECODE_NOALLOC_BYTES (8u << 20)
int gpt_decode_step_noalloc(const gpt_config* cfg, const void* params, const int32_t* tok, int B, int32_t* pos,
                            void* k_cache, void* v_cache, int Tmax, int32_t* next_tok, void* logits,
                            void* stream);

/* ---- sampling the next token from rows of logits ----
 * Steps, in this order (the pages name them; the order is a reading):
 *   repetition penalty ("02 GPT 架构" §8.4): the logit of a token whose bit is
 *     set in `seen` is divided by the penalty when positive, multiplied by it
 *     when negative;
 *   temperature ("预训练一个 Mini GPT" 第7步; "02 GPT 架构" §8.1): key = z'/T;
 *     T <= 0 selects the greedy choice (largest penalised logit, lowest index);
 *   top-k ("02 GPT 架构" §8.2; "GPT-1学习笔记" §6.2): the k most probable;
 *   top-p ("02 GPT 架构" §8.3; "GPT-1学习笔记" §6.2): of those, the smallest
 *     most-probable prefix whose renormalised mass reaches p;
 *   draw ("预训练一个 Mini GPT" 第7步): the first candidate, in the order of
 *     descending weight (equal weights: ascending index), whose cumulative
 *     mass exceeds u times the mass of the candidates.
 * Weights are exp(key - max key) evaluated in double and rounded once to
 * float; masses are double sums of them.  Deterministic: the same inputs give
 * the same tokens (no atomics decide a value). */
typedef struct gpt_sampling {
  float temperature;          /* <= 0: greedy */
  int32_t top_k;              /* <= 0 or >= V: no top-k */
  float top_p;                /* in (0, 1]; 1: no top-p */
  float repetition_penalty;   /* > 0; 1: no penalty */
} gpt_sampling;

/* Samples one token per row.
 *   logits   (device) [B, V] in cfg->dtype, row stride V.
 *   s        (host) sampling settings, checked before any launch.
 *   u        (device) float [B], uniforms in [0, 1), one per row (the caller's
 *            random stream); may be NULL when s->temperature <= 0.
 *   seen     (device, nullable) uint32 [B][(V + 31) / 32] bit sets: bit i of
 *            row b marks token i as already present in sequence b.  Read for
 *            the penalty; the chosen token's bit is set.
 *   next_tok (device) int32 [B].
 * Requires V <= 53248 (GPT_ERR_CONFIG otherwise) and B >= 1.  No workspace. */
int gpt_sample(const gpt_config* cfg, const void* logits, int B, const gpt_sampling* s, const float* u,
               uint32_t* seen, int32_t* next_tok, void* stream);

/* Sets the bits of tokens (device, int32 [B, T]; ids outside [0, V) are
 * ignored) in seen (device, uint32 [B][(V + 31) / 32]); bits already set stay. */
int gpt_mark_seen(const gpt_config* cfg, const int32_t* tokens, int B, int T, uint32_t* seen, void* stream);

/* ---- backward of the loss through the head ----
 * A training step back-propagates the mean next-token cross-entropy to every
 * parameter ("预训练一个 Mini GPT（1.24 亿参数）", 训练循环).  The loss
 * gradient of the logits is (softmax(z) - onehot(y)) / n_valid on rows with a
 * target and 0 elsewhere (n_valid = number of rows with a target); with a tied
 * head the token table's gradient is the sum of the head's share and the
 * lookup's share ("第 25 章 从小 GPT 到 GPT-2" §25.4): gpt_head_backward adds
 * the first, gpt_embedding_backward the second.
 *
 * Gradients are fp32 in a blob laid out like the parameter blob
 * (gpt_param_offsets, gpt_param_count elements) and are ACCUMULATED (+=):
 * the caller zeroes the blob at the start of a step.  Products use the
 * compute dtype (cfg->dtype) with fp32 accumulation; dz is rounded to it
 * before the two gradient products. */

/* Device workspace bytes of gpt_head_backward for a [B, T] batch (host only).
 * Requires B * T <= 2^20. */
int gpt_head_backward_workspace_bytes(const gpt_config* cfg, int B, int T, size_t* bytes);

/* From the rows the final LayerNorm reads (pre-LN models) or the final hidden
 * rows themselves (post-LN models) to the loss:
 *   params     (device) parameter blob in cfg->dtype.
 *   idx        (device) int32 [B, T]: only used to derive targets when
 *              targets is NULL (same rule as gpt_forward).
 *   targets    (device, nullable) int32 [B, T]; -1 (or an id outside [0, V))
 *              = no target.
 *   x          (device) fp32 [B*T, C] (the residual stream after the last
 *              block; read only).
 *   dx         (device) fp32 [B*T, C]: d loss / d x, overwritten.
 *   grads      (device) fp32 gradient blob: += the head matrix's gradient
 *              (the token table's head share when tied, head_w when untied)
 *              and, for pre-LN models, lnf_g / lnf_b.
 *   mean_loss  (device, nullable) fp32 [1]: the loss itself (as gpt_forward).
 *   ws         (device) at least gpt_head_backward_workspace_bytes.
 * The logits are recomputed twice (row log-sum-exp, then dz from fp32
 * accumulators) and never stored.  Requires 1 <= T <= ctx, B * T <= 2^20.
 * No position with a target: every gradient added is 0 (mean_loss NaN).
 * GPT-2 blocks only (arch 1: GPT_ERR_CONFIG). */
int gpt_head_backward(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                      const int32_t* targets, const float* x, float* dx, float* grads, float* mean_loss, void* ws,
                      size_t ws_bytes, void* stream);

/* Embedding backward, x0[b, t] = wte[idx[b, t]] + wpe[t]:
 *   grads[wte row v] += sum of dx0 over the positions holding v (position
 *   order), grads[wpe row t] += sum over the batch of dx0[:, t].
 *   idx  (device) int32 [B, T]; a position holding an id outside [0, V)
 *        adds nothing to the token table (its position row still gets dx0;
 *        arch 1 models have no position table). 
 *   dx0  (device) fp32 [B*T, C]: d loss / d x0.
 * Requires 1 <= T <= ctx, B * T <= 2^24.  No workspace. */
int gpt_embedding_backward(const gpt_config* cfg, const int32_t* idx, int B, int T, const float* dx0, float* grads,
                           void* stream);

/* ---- backward of the blocks (pre-LN GPT-2 blocks: arch 0, post_ln 0) ----
 * A whole gradient of the mean loss: gpt_forward_train (each block's input
 * residual; with a null mean_loss the head is left to the next step),
 * gpt_head_backward on xs[L] (which also gives the loss), gpt_block_backward for
 * l = L-1 .. 0 (each turns d loss / d(block l's output) into d loss / d(its
 * input)), then gpt_embedding_backward on the last dx.  Blocks are recomputed
 * from their inputs (only the L+1 residual rows are kept between the passes). */

/* The forward pass and mean loss (no logits), writing xs (device, fp32
 * [L+1][B*T][C]): xs[l] = the residual entering block l, xs[L] = the rows
 * the final LayerNorm reads.  mean_loss (device, one float) may be null:
 * then the final LayerNorm, the head and the loss are skipped (a gradient
 * computation gets the same loss from gpt_head_backward).  Same workspace as
 * gpt_forward.  B*T <= 2^20. */
int gpt_forward_train(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                      const int32_t* targets, float* xs, float* mean_loss, void* ws, size_t ws_bytes, void* stream);

/* Device workspace bytes of gpt_block_backward for a [B, T] batch (host only). */
int gpt_block_backward_workspace_bytes(const gpt_config* cfg, int B, int T, size_t* bytes);

/* Backward of block `layer` (0 <= layer < L): out = x1 + mlp(LN2(x1)),
 * x1 = x + attn(LN1(x)).
 *   x      (device) fp32 [B*T, C]: the block's input (read only).
 *   dy     (device) fp32 [B*T, C]: d loss / d out (read only).
 *   dx     (device) fp32 [B*T, C]: d loss / d x, overwritten (must not alias
 *          x or dy).
 *   grads  (device) fp32 gradient blob: += this block's twelve tensors.
 * The block's forward is recomputed with the forward kernels; the products
 * run on bf16 (or fp32) operands with fp32 accumulation.  Attention's
 * gradient keeps each head's P^T, dS = P (dP - dO.O) / sqrt(D) and dS^T
 * ([B*H][T][Tp] in the workspace; bf16: P^T comes straight from the q.k
 * product with the recomputed forward's row log-sum-exp, dS from the dO.u
 * product, so the scores and dP are never stored; fp32: S and dP are stored
 * and row kernels form P and dS) and runs the contractions as batched
 * matrix-core products.  B*T <= 2^20. */
int gpt_block_backward(const gpt_config* cfg, const void* params, int layer, int B, int T, const float* x,
                       const float* dy, float* dx, float* grads, void* ws, size_t ws_bytes, void* stream);

/* Human-readable text for a status code (static storage). */
const char* gpt_status_string(int status);

/* ---- single-operation entry points (same conventions), used to check each
 * kernel on its own against the oracle ---- */

/* out[M,C] = LN(x[M,C]; g, b, eps) in cfg->dtype; x fp32 (device). */
int gpt_debug_layernorm(const gpt_config* cfg, const float* x, const void* g, const void* b, int M,
                        void* out, void* stream);

/* out[M,N] = act(A[M,K] W[N,K]^T + bias[N]); A, W, bias in cfg->dtype (bias
 * nullable); act 0 = none, 1 = tanh GELU, 2 = exact GELU; out fp32 if out_f32 else cfg->dtype.
 * Requires K % 8 == 0 (bf16) or K % 4 == 0 (fp32). */
int gpt_debug_linear(const gpt_config* cfg, const void* A, const void* W, const void* bias, int M, int N,
                     int K, int act, int out_f32, void* out, void* stream);

/* Causal attention of every (b, h) ("第 25 章 从小 GPT 到 GPT-2" §25.2):
 * q, k, u [B,H,T,D] in cfg->dtype; out [B*T, C] in cfg->dtype with head h in
 * columns [hD, hD+D) (heads merged back). */
int gpt_debug_attention(const gpt_config* cfg, const void* q, const void* k, const void* u,
                        int B, int T, void* out, void* stream);

/* The same attention on token-major rows, the layout the forward's c_attn
 * writes: qkv [B*T, 3C] in cfg->dtype, row t of sequence b holding q | k | u
 * (head h in columns [hD, hD+D) of each third); out [B*T, C] as above.
 * Errors: GPT_ERR_NULL for a null pointer, GPT_ERR_SHAPE for B or T <= 0. */
int gpt_debug_attention_rows(const gpt_config* cfg, const void* qkv, int B, int T, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPTMI_H */
