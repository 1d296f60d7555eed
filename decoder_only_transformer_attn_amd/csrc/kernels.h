// Internal launcher interface between the host API (gptmi.cpp) and the HIP
// kernels.  Every launcher enqueues on the given stream and returns the launch
// status; none allocates or synchronises.  dtype: 0 = fp32, 1 = bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptmi {

struct QKVArgs {
  const void* A;      // normalised rows [M, C]
  const void* W;      // weight [(H + 2 Hkv) D, C]: rows of W_q, W_k, W_v
  const void* bias;   // [(H + 2 Hkv) D], nullable (no bias)
  int M, C, H, D, T_seq;
  void* q; long long q_bh;             // Q [B,H,T,D]
  void* k; long long k_bh;             // K [B,Hkv,Tk,D]
  void* v; long long v_bh;             // U [B,Hkv,Tk,D]
  const int32_t* pos;                  // nullable: cache position of t = 0
  int Tk;                              // K/U rows available; writes at positions >= Tk are dropped
  int Hkv;                             // K/U heads (= H without grouping)
  const float2* rope;                  // nullable: (cos, sin) [positions][D/2]; rotates Q and K pairs
};
// (cos, sin) of p * theta^(-2i/D) for p < rows, i < D/2, in double, rounded to float.
hipError_t launch_rope_table(float2* tab, int rows, int D, double theta, hipStream_t st);

// Embedding (+ first LayerNorm) or LayerNorm of M rows.
struct LnArgs {
  int M, C, T_seq;
  float eps;
  const int32_t* idx;                  // embedding: token ids [M]
  const void* wte; const void* wpe;    // embedding tables
  int vocab, ctx;
  const int32_t* pos;                  // embedding: nullable device position added to t
  float* x;                            // residual [rows, C]: written by the embedding, read by LayerNorm
  int in_mul, in_add;                  // LayerNorm input row = row * in_mul + in_add
  const void* g; const void* b;        // LayerNorm gain / bias
  void* out;                           // [M, C] normalised rows
  int* zero; int zero_n;               // embedding: nullable ints set to zero (split-K counters)
  int ident;                           // embedding: out = x itself (no LayerNorm; post-LN models)
  int write_x;                         // LayerNorm: the normalised row also replaces its x row (post-LN)
  int rms;                             // RMSNorm: no mean centring (b is then NULL: no bias)
  // residual LayerNorm (launch_resid_layernorm): x += sum of the nsplit fp32
  // slices part[s][M][C] (slice order) + rbias, then the LayerNorm of the new x
  const float* part; int nsplit; const void* rbias;
  // ... and pf_blocks[r] more blocks per byte range pf[r] (r = 0, 1; the
  // next products' weights, resid_ln_prefetch_blocks(pf_bytes[r]) blocks)
  // that read it so that those products find it cached; the words read are
  // folded into one value stored only through pf_sink (null in the library:
  // it only keeps the loads from being dropped)
  const void* pf[2]; size_t pf_bytes[2]; int pf_blocks[2]; uint32_t* pf_sink;
};

// Attention of one new query per (b, h) over positions 0 .. *pos of the cache.
struct DecAttnArgs {
  const void* q;                       // [B, H, D]
  const void* k; const void* v;        // this layer's caches [B, Hkv, Tmax, D]
  long long kv_bh;                     // Tmax * D
  int Tmax;
  const int32_t* pos;                  // device
  void* o; int o_ld;                   // [B, o_ld], head h at columns [hD, hD+D)
  int B, H, D;
  float scale_log2;
  int Hkv;                             // cache heads; query head h reads head h / (H / Hkv)
  int alibi;                           // 1: scores carry -m_h (pos - j), m_h = 2^(-8 (h+1) / H)
};

struct AttnArgs {
  // element (b, h, t, d) of Q at q[b q_sb + h q_sh + t q_st + d]; K and U
  // likewise with their head hk = h / (H / Hkv).  Head-major [B,H,T,D]:
  // (sb, sh, st) = (H T D, T D, D); token-major rows of the fused QKV product
  // [B*T, C + 2 Hkv D]: (T (C + 2 Hkv D), D, C + 2 Hkv D).
  const void* q; long long q_sb, q_sh; int q_st;
  const void* k; long long k_sb, k_sh; int k_st;
  const void* v; long long v_sb, v_sh; int v_st;
  void* o; int o_ld;                   // O [B*T, o_ld], head h at columns [hD, hD+D)
  int B, H, T_seq, D;
  int Hkv;                             // K/U heads; query head h reads K/U head h / (H / Hkv)
  float scale_log2;                    // log2(e) / sqrt(D)
  int alibi;                           // 1: scores carry -m_h (t - j), m_h = 2^(-8 (h+1) / H)
  float* lse2;                         // optional [B*H][T]: log2 of each row's softmax denominator
                                       // (the log-sum-exp of the scaled scores, in log2 units)
};

// Q, K and U stored head-major: element (b, h, t, d) at base + (b Hx + h) bh + t D + d.
inline void attn_headmajor(AttnArgs& a, const void* q, long long q_bh, const void* k, const void* v, long long kv_bh,
                           int H, int Hkv, int D) {
  a.q = q; a.q_sh = q_bh; a.q_sb = q_bh * H; a.q_st = D;
  a.k = k; a.k_sh = kv_bh; a.k_sb = kv_bh * Hkv; a.k_st = D;
  a.v = v; a.v_sh = kv_bh; a.v_sb = kv_bh * Hkv; a.v_st = D;
}

// Split-K scratch of the skinny (M <= 64) bf16 products: per-column-tile
// arrival counters, which must be zero when a product starts and are zero
// again when it ends, and fp32 partial tiles of 64 x 32 (8 KB each).  With
// a null pointer (or too little room) the products run without split-K.
struct SkinnyWs {
  float* part; int part_tiles;
  int* cnt; int cnt_len;
};

hipError_t launch_embed_ln(int dtype, const LnArgs& a, hipStream_t st);
hipError_t launch_layernorm(int dtype, const LnArgs& a, hipStream_t st);
// bf16 only, at most 12 slices: the residual update of a split product
// followed by the LayerNorm that reads it (one row per block).
hipError_t launch_resid_layernorm(const LnArgs& a, hipStream_t st);
int resid_ln_prefetch_blocks(size_t nbytes);
hipError_t launch_linear(int dtype, const void* A, int lda, const void* W, int ldw, const void* bias, int M, int N,
                         int K, void* out, int ldo, int act, int out_f32, hipStream_t st,
                         const SkinnyWs* sk = nullptr);
hipError_t launch_linear_resid(int dtype, const void* A, int lda, const void* W, int ldw, const void* bias, int M,
                               int N, int K, float* x, int ldx, hipStream_t st, const SkinnyWs* sk = nullptr);
// bf16 products of at most 64 rows with K split into S slices (K / S one of
// 128, 256, 384, 512, 768; rows contiguous): slice s is written as the raw
// fp32 partial product part[s][M][N] (S M N <= part_floats), no bias.
hipError_t launch_skinny_slices(const void* A, const void* W, int M, int N, int K, int S, float* part,
                                size_t part_floats, hipStream_t st);
hipError_t launch_qkv(int dtype, const QKVArgs& a, hipStream_t st, const SkinnyWs* sk = nullptr);
hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st);
// Vocabulary tiles of the head's partials for M rows (CE or argmax mode).
int head_ntiles(int dtype, int M, int V, int C, bool argmax);
// Tied head over M token rows.  CE mode (part_idx == NULL): softmax partials
// and target logits for the next-token loss.  Argmax mode (part_idx != NULL):
// per-(row, N-tile) maximum and its lowest index; part_sum/tgt unused.
hipError_t launch_head_ce(int dtype, const void* A, const void* wte, int M, int V, int C, void* logits,
                          long long ld_logits, float* part_max, float* part_sum, float* tgt, int32_t* part_idx,
                          const int32_t* targets, const int32_t* idx, int T_seq, hipStream_t st);
// Greedy choice per row from the head's argmax partials (lowest index wins
// ties); then *pos = set_pos if set_pos >= 0, else *pos += 1 (if pos).
hipError_t launch_argmax_reduce(int M, int ntiles, const float* part_max, const int32_t* part_idx, int32_t* next_tok,
                                int32_t* pos, int set_pos, hipStream_t st);
hipError_t launch_attention_decode(int dtype, const DecAttnArgs& a, hipStream_t st);
// bf16, Hkv = H, no ALiBi: the decode attention fed by the S K-slices of the
// Q|K|U product (part[s][B][3C], fp32, no bias); appends k and u at *pos.
hipError_t launch_attention_decode_slices(const DecAttnArgs& a, const float* part, int S, const void* bias,
                                          hipStream_t st);
// Next-token sampling of B rows of logits (one block per row).
struct SampleArgs {
  const void* logits; long long ld;    // [B, ld] in the compute dtype, V valid columns
  int V, B;
  float temperature;                   // <= 0: greedy
  int top_k;                           // <= 0 or >= V: off
  float top_p;                         // >= 1: off (> 0)
  float penalty;                       // repetition penalty (1: off)
  const float* u;                      // [B] uniforms in [0, 1)
  uint32_t* seen;                      // nullable [B, seen_words] bit sets; the chosen token's bit is set
  int seen_words;
  int32_t* out;                        // [B]
};
hipError_t launch_sample(int dtype, const SampleArgs& a, hipStream_t st);
hipError_t launch_mark_seen(const int32_t* tokens, int B, int T, int V, uint32_t* seen, hipStream_t st);
// Per-token loss from the head partials, then a deterministic mean.
int ce_reduce_blocks(int M);
// Backward of the loss through the head, the final LayerNorm and the embeddings.
hipError_t launch_head_dz(int dtype, const void* A, const void* W, int M, int V, int C, const float* lse,
                          const int32_t* y, const float* inv, void* dz, long long ld, void* dzT, long long ldT,
                          hipStream_t st);
hipError_t launch_gemm_f32out(int dtype, const void* A, int lda, const void* W, int ldw, int M, int N, int K,
                              float* out, int ldo, int accumulate, hipStream_t st);
hipError_t launch_bwd_rows(int M, int ntiles, const float* part_max, const float* part_sum, const int32_t* targets,
                           const int32_t* idx, int T_seq, int V, float* lse, int32_t* yv, float* inv, hipStream_t st);
hipError_t launch_transpose(int dtype, const void* in, long long ld_in, int R, int Cc, void* out, int Rp,
                            hipStream_t st);
hipError_t launch_zero_cols(int dtype, void* p, long long ld, int R, int c0, int c1, hipStream_t st);
hipError_t launch_cast_rows(int dtype, const float* x, long long n, void* out, hipStream_t st);
// in fp32 [R, Cc] (dense) -> out_rm [R, Cc] and its transpose out_t [Cc, Rp] (zero-padded), compute dtype
hipError_t launch_cast_transpose(int dtype, const float* in, int R, int Cc, void* out_rm, void* out_t, int Rp,
                                 hipStream_t st);
int ln_bwd_chunks(int M);
hipError_t launch_ln_backward(int dtype, int M, int C, const float* x, const void* g, const float* dy, float eps,
                              float* dx, float* mu, float* rs, float* part, float* dg, float* db, hipStream_t st,
                              int accumulate);
// Per-(b, h) operand offsets of a batched product: b * (.b) + h * (.h), z = b * H + h.
struct BatchStrides { long long ab, ah, wb, wh, ob, oh; int H; };
hipError_t launch_gemm_batched(int dtype, const void* A, int lda, const void* W, int ldw, int M, int N, int K,
                               float* out, int ldo, const BatchStrides& bs, int Z, hipStream_t st, int causal = 0);
// Split-K partials: out + z zstride [M, N] = A[:, z Ks, +Ks) . W[:, z Ks, +Ks)^T, z < S.
hipError_t launch_gemm_f32_splitk(int dtype, const void* A, int lda, const void* W, int ldw, int M, int N, int Ks,
                                  int S, float* out, long long zstride, hipStream_t st);
// Attention backward scratch: S / dP fp32 [B*H][T][Tp]; P, P^T, dS, dS^T [B*H][T][Tp];
// dO in the compute dtype [B*T][C]; per-head transposes of dO, K, Q [B*H][D][Tp].
// With lse2 (from the forward pass), O and Dv set, the bf16 path fuses the
// softmax into the score product and dS into the dP product (S and dP are
// then never stored): Dv [B*H][T] receives the rows' dO . O.
struct AttnBwdWs {
  float* S; void* P; void* PT; void* dS; void* dST; void* doc; void* dOT; void* KT; void* QT; int Tp;
  const float* lse2; const void* o; float* Dv;
};
hipError_t launch_attn_scores_bwd(int mode, const void* A, int lda, const void* W, int ldw, int Tn, int D,
                                  const BatchStrides& bs, int Z, const float* rowv, const void* PT, void* out,
                                  void* outT, int ld, float sc, hipStream_t st);
hipError_t launch_attention_backward(int dtype, const void* q, const void* k, const void* u, const float* dout,
                                     float* dqkv, int B, int H, int T, int D, const AttnBwdWs& w, hipStream_t st);
hipError_t launch_act_fwd(int dtype, const void* u, long long n, int act, void* h, hipStream_t st);
hipError_t launch_act_bwd(int dtype, float* d, const void* u, long long n, int act, void* dc, hipStream_t st);
// out[c] += sum over rows of a[M, N]; part holds max(colsum_chunks(M), ln_bwd_chunks(M)) * N floats
int colsum_chunks(int M);
hipError_t launch_colsum(int M, int N, const float* a, float* part, float* out, hipStream_t st);
// out += (accumulate) or = the S slices part[z n, +n) summed in slice order
hipError_t launch_add_partials(float* out, const float* part, long long n, int S, hipStream_t st, int accumulate = 1);
hipError_t launch_embed_backward(const int32_t* idx, int B, int T, int C, int V, const float* dx0, float* dwte,
                                 float* dwpe, hipStream_t st);
hipError_t launch_ce_reduce(int M, int ntiles, const float* part_max, const float* part_sum, const float* tgt,
                            const int32_t* targets, const int32_t* idx, int T_seq, int V, float* token_loss,
                            double* block_sums, float* mean_loss, hipStream_t st);

}  // namespace gptmi
