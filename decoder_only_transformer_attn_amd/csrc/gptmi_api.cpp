// Host side of the C ABI declared in include/gptmi.h: validation, parameter
// blob offsets, workspace plan and the launch sequences of the forward pass,
// the prefill and the decode step.  Stateless: every call validates on the
// host, then enqueues kernels on the caller's stream and returns without
// synchronising.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/gptmi.h"
#include "kernels.h"

using namespace gptmi;

namespace {

// (the library keeps no state between calls: a failed HIP call is reported
// as GPT_ERR_HIP only, without its HIP code)
int hip_status(hipError_t e) { return e == hipSuccess ? GPT_OK : GPT_ERR_HIP; }

#define GPT_TRY(expr)                       \
  do {                                      \
    int _s = hip_status(expr);              \
    if (_s != GPT_OK) return _s;            \
  } while (0)

int vec_of(const gpt_config* c) { return c->dtype == GPT_BF16 ? 8 : 4; }
size_t esize(const gpt_config* c) { return c->dtype == GPT_BF16 ? 2 : 4; }

int check_config(const gpt_config* c) {
  if (!c) return GPT_ERR_NULL;
  if (c->dtype != GPT_F32 && c->dtype != GPT_BF16) return GPT_ERR_DTYPE;
  if (c->vocab <= 0 || c->ctx <= 0 || c->n_embd <= 0 || c->n_head <= 0 || c->n_layer < 0 || c->n_ff <= 0)
    return GPT_ERR_CONFIG;
  if (!(c->ln_eps > 0.f) || !std::isfinite(c->ln_eps)) return GPT_ERR_CONFIG;
  if ((c->activation != 0 && c->activation != 1) || (c->post_ln != 0 && c->post_ln != 1) ||
      (c->untied_head != 0 && c->untied_head != 1))
    return GPT_ERR_CONFIG;
  if (c->n_embd % c->n_head != 0) return GPT_ERR_CONFIG;
  const int D = c->n_embd / c->n_head, v = vec_of(c);
  if (c->n_embd % v || c->n_ff % v || D % v || D > 128 || c->n_embd > 2048) return GPT_ERR_CONFIG;
  if (c->arch != 0 && c->arch != 1) return GPT_ERR_CONFIG;
  if (c->alibi != 0 && (c->alibi != 1 || c->arch != 1)) return GPT_ERR_CONFIG;   // LLaMA-style blocks only
  if (c->arch == 1) {
    // the GPT-2 variant flags do not apply to LLaMA-style blocks
    if (c->activation != 0 || c->post_ln != 0) return GPT_ERR_CONFIG;
    if (c->n_kv_head < 0 || c->n_kv_head > c->n_head || (c->n_kv_head > 0 && c->n_head % c->n_kv_head != 0))
      return GPT_ERR_CONFIG;
    if (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta)) return GPT_ERR_CONFIG;
  } else if (c->n_kv_head != 0 && c->n_kv_head != c->n_head) {
    return GPT_ERR_CONFIG;
  }
  return GPT_OK;
}

int kv_heads(const gpt_config* c) { return c->n_kv_head > 0 ? c->n_kv_head : c->n_head; }

int64_t offsets(const gpt_config* c, int64_t* out, int n) {
  const int64_t V = c->vocab, C = c->n_embd, F = c->n_ff, ctx = c->ctx;
  int64_t off = 0;
  int k = 0;
  auto put = [&](int64_t size) {
    if (out && k < n) out[k] = off;
    ++k;
    off += size;
  };
  put(V * C);
  if (c->arch == 1) {   // LLaMA-style: no position table, no biases, one final RMSNorm gain
    const int64_t KV = (int64_t)kv_heads(c) * (C / c->n_head);
    for (int l = 0; l < c->n_layer; ++l) {
      put(C); put((C + 2 * KV) * C); put(C * C); put(C); put(2 * F * C); put(C * F);
    }
    put(C);
    if (c->untied_head) put(V * C);
    if (out && k < n) out[k] = off;
    return off;
  }
  put(ctx * C);
  for (int l = 0; l < c->n_layer; ++l) {
    put(C); put(C); put(3 * C * C); put(3 * C); put(C * C); put(C);
    put(C); put(C); put(F * C); put(F); put(C * F); put(C);
  }
  if (!c->post_ln) {   // final LayerNorm
    put(C);
    put(C);
  }
  if (c->untied_head) put(V * C);
  if (out && k < n) out[k] = off;
  return off;
}

int offset_count(const gpt_config* c) {
  if (c->arch == 1) return 1 + 6 * c->n_layer + 1 + (c->untied_head ? 1 : 0) + 1;
  return 2 + 12 * c->n_layer + (c->post_ln ? 0 : 2) + (c->untied_head ? 1 : 0) + 1;
}

// Element offsets of the tensors of one layer, packing order as documented.
struct LayerP { int64_t ln1_g, ln1_b, attn_w, attn_b, proj_w, proj_b, ln2_g, ln2_b, fc_w, fc_b, fcproj_w, fcproj_b; };

// LLaMA-style models use the same fields: ln1_g / ln2_g are the RMSNorm gains,
// attn_w the stacked W_q|W_k|W_v, proj_w W_o, fc_w the interleaved gate/up
// rows, fcproj_w the down projection; the biases are absent (-1).
struct Params {
  const char* base;
  size_t es;
  int64_t C, F, V, ctx, L;
  bool post_ln, untied;
  int arch;
  int64_t KV;   // K/V width Hkv * D
  const void* at(int64_t e) const { return base + e * (int64_t)es; }
  const void* opt(int64_t e) const { return e < 0 ? nullptr : at(e); }
  int64_t layer_base(int l) const {
    if (arch == 1) return V * C + (int64_t)l * (2 * C + (C + 2 * KV) * C + C * C + 3 * F * C);
    return V * C + ctx * C + (int64_t)l * (4 * C * C + 4 * C + 2 * C * F + F + C + 4 * C);
  }
  LayerP layer(int l) const {
    LayerP r;
    if (arch == 1) {
      r.ln1_g = layer_base(l);
      r.attn_w = r.ln1_g + C;
      r.proj_w = r.attn_w + (C + 2 * KV) * C;
      r.ln2_g = r.proj_w + C * C;
      r.fc_w = r.ln2_g + C;
      r.fcproj_w = r.fc_w + 2 * F * C;
      r.ln1_b = r.attn_b = r.proj_b = r.ln2_b = r.fc_b = r.fcproj_b = -1;
      return r;
    }
    r.ln1_g = layer_base(l);
    r.ln1_b = r.ln1_g + C;
    r.attn_w = r.ln1_b + C;
    r.attn_b = r.attn_w + 3 * C * C;
    r.proj_w = r.attn_b + 3 * C;
    r.proj_b = r.proj_w + C * C;
    r.ln2_g = r.proj_b + C;
    r.ln2_b = r.ln2_g + C;
    r.fc_w = r.ln2_b + C;
    r.fc_b = r.fc_w + F * C;
    r.fcproj_w = r.fc_b + F;
    r.fcproj_b = r.fcproj_w + C * F;
    return r;
  }
  int64_t lnf_g() const { return layer_base((int)L); }   // pre-LN (or the final RMSNorm gain)
  int64_t lnf_b() const { return arch == 1 ? -1 : layer_base((int)L) + C; }
  int64_t wpe() const { return arch == 1 ? -1 : V * C; }
  // the head matrix: the token table, or the tensor after the last layer (and the final norm)
  int64_t head_w() const {
    if (!untied) return 0;
    if (arch == 1) return layer_base((int)L) + C;
    return layer_base((int)L) + (post_ln ? 0 : 2 * C);
  }
};

Params params_of(const gpt_config* c, const void* p) {
  return Params{static_cast<const char*>(p), esize(c), c->n_embd, c->n_ff, c->vocab, c->ctx, c->n_layer,
                c->post_ln != 0, c->untied_head != 0, c->arch,
                (int64_t)kv_heads(c) * (c->n_embd / c->n_head)};
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace of a [B, T] pass.  Decode calls keep K/U in the caller's caches
// and run the head on B rows only; they add a_last [B, C] and the argmax
// partial indices.  Passes of at most 64 bf16 rows (decode steps) add the
// split-K scratch of the skinny products.
struct Plan {
  size_t x, a, q, k, v, o, h, pmax, psum, tgt, tok, bsum, alast, pidx, skpart, skcnt, rope, total;
  int ntiles, nblocks;
};

constexpr int SK_PART_TILES = 512;   // 64 x 32 fp32 partial tiles (4 MB)
constexpr int SK_COUNTERS = 256;     // column tiles of 32 (N <= 8192)

Plan plan(const gpt_config* c, int B, int T, bool decode) {
  Plan p{};
  const size_t M = (size_t)B * T, C = c->n_embd, F = c->n_ff, es = esize(c);
  const size_t head_rows = decode ? (size_t)B : M;
  p.ntiles = head_ntiles(c->dtype, (int)head_rows, c->vocab, c->n_embd, decode);
  p.nblocks = ce_reduce_blocks((int)M);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  p.x = take(M * C * 4);
  p.a = take(M * C * es);
  const size_t KV = (size_t)kv_heads(c) * (C / c->n_head);
  if (decode) {
    p.q = take(M * C * es);
  } else {
    // one region [M, C + 2 KV]: token-major rows of the fused Q|K|U product
    // (GPT-2 forward), or head-major Q, K and U one after another
    p.q = take(M * (C + 2 * KV) * es);
    p.k = p.q + M * C * es;
    p.v = p.k + M * KV * es;
  }
  p.o = take(M * C * es);
  p.h = take(M * F * es);
  p.pmax = take(head_rows * p.ntiles * 4);
  p.psum = decode ? 0 : take(head_rows * p.ntiles * 4);
  p.tgt = decode ? 0 : take(M * 4);
  p.tok = decode ? 0 : take(M * 4);
  p.bsum = decode ? 0 : take((size_t)p.nblocks * 2 * 8);
  p.alast = decode ? take((size_t)B * C * es) : 0;
  p.pidx = decode ? take((size_t)B * p.ntiles * 4) : 0;
  const bool split = M <= 64 && c->dtype == GPT_BF16;
  p.skpart = split ? take((size_t)SK_PART_TILES * 64 * 32 * 4) : 0;
  p.skcnt = split ? take((size_t)SK_COUNTERS * 4) : 0;
  p.rope = c->arch == 1 ? take((size_t)c->ctx * (C / c->n_head / 2) * 8) : 0;
  p.total = off;
  return p;
}

template <typename P> P* at(void* base, size_t off) { return reinterpret_cast<P*>(static_cast<char*>(base) + off); }

// How a pass stores K/U and attends:
//   FORWARD: K/U of the batch in the workspace, causal flash attention;
//   PREFILL: K/U written to the cache at positions 0..T-1, flash attention on the cache;
//   STEP:    T = 1, K/U appended to the cache at *pos, one-query attention over the cache.
enum Mode { FORWARD, PREFILL, STEP };

struct Pass {
  const gpt_config* cfg;
  Params P;
  const int32_t* idx;
  int B, T;
  Mode mode;
  const int32_t* pos;        // STEP: device position of the new token
  void* kc; void* vc;        // PREFILL / STEP caches [L][B][H][Tmax][D]
  int Tmax;
  void* ws;
  Plan pl;
  hipStream_t st;
  void* ev_begin; void* ev_end; int which;   // timing hook
  float* xs;                 // nullable: each block's input residual [L+1][M][C] (the last: ln_f's input)
};

hipError_t mark(const Pass& s, int kind, bool last_layer, bool begin) {
  if (kind != s.which || !last_layer) return hipSuccess;
  void* ev = begin ? s.ev_begin : s.ev_end;
  return ev ? hipEventRecord(static_cast<hipEvent_t>(ev), s.st) : hipSuccess;
}

// LLaMA-style embedding and blocks ("02 GPT 架构" §6.1-6.3): token rows only,
// then per block RMSNorm -> W_q|W_k|W_v with RoPE on Q and K (angle table in
// the workspace) -> grouped-query attention -> W_o + residual -> RMSNorm ->
// gate/up product with the SwiGLU epilogue -> down projection + residual.
// Leaves the residual stream in ws.x (with no blocks ws.a holds the final
// RMSNorm of the embedding).
int run_blocks_llama(const Pass& s) {
  const gpt_config* cfg = s.cfg;
  const Params& P = s.P;
  const int dt = cfg->dtype, B = s.B, T = s.T, M = B * T, C = cfg->n_embd, F = cfg->n_ff;
  const int H = cfg->n_head, D = C / H, L = cfg->n_layer, Hkv = kv_heads(cfg);
  float* x = at<float>(s.ws, s.pl.x);
  void* a = at<char>(s.ws, s.pl.a);
  void* q = at<char>(s.ws, s.pl.q);
  void* o = at<char>(s.ws, s.pl.o);
  void* h = at<char>(s.ws, s.pl.h);
  const size_t es = esize(cfg);
  const long long cache_layer = (long long)B * Hkv * s.Tmax * D;
  SkinnyWs skw{};
  if (s.pl.skpart) skw = SkinnyWs{at<float>(s.ws, s.pl.skpart), SK_PART_TILES, at<int>(s.ws, s.pl.skcnt), SK_COUNTERS};
  const SkinnyWs* sk = s.pl.skpart ? &skw : nullptr;
  const int alibi = cfg->alibi;   // ALiBi: no rotation, a distance bias in the attention scores
  float2* rope = alibi ? nullptr : at<float2>(s.ws, s.pl.rope);
  if (!alibi) GPT_TRY(launch_rope_table(rope, cfg->ctx, D, (double)cfg->rope_theta, s.st));

  LnArgs la{};
  la.M = M; la.C = C; la.T_seq = T; la.eps = cfg->ln_eps; la.rms = 1;
  la.idx = s.idx; la.wte = P.at(0); la.wpe = nullptr; la.vocab = cfg->vocab; la.ctx = cfg->ctx;
  la.pos = s.mode == STEP ? s.pos : nullptr;
  la.x = x; la.in_mul = 1; la.in_add = 0;
  la.g = P.at(L > 0 ? P.layer(0).ln1_g : P.lnf_g()); la.b = nullptr;
  la.out = a;
  la.zero = sk ? skw.cnt : nullptr; la.zero_n = sk ? skw.cnt_len : 0;
  GPT_TRY(launch_embed_ln(dt, la, s.st));
  la.idx = nullptr; la.pos = nullptr; la.zero = nullptr; la.zero_n = 0;

  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  for (int l = 0; l < L; ++l) {
    const LayerP w = P.layer(l);
    const bool last = l == L - 1;
    void* kbuf = s.mode == FORWARD ? at<char>(s.ws, s.pl.k) : static_cast<char*>(s.kc) + l * cache_layer * es;
    void* vbuf = s.mode == FORWARD ? at<char>(s.ws, s.pl.v) : static_cast<char*>(s.vc) + l * cache_layer * es;
    const long long kv_bh = s.mode == FORWARD ? (long long)T * D : (long long)s.Tmax * D;
    QKVArgs qa{};
    qa.A = a; qa.W = P.at(w.attn_w); qa.bias = nullptr;
    qa.M = M; qa.C = C; qa.H = H; qa.D = D; qa.T_seq = T;
    qa.q = q; qa.q_bh = (long long)T * D;
    qa.k = kbuf; qa.k_bh = kv_bh;
    qa.v = vbuf; qa.v_bh = kv_bh;
    qa.pos = s.mode == STEP ? s.pos : nullptr;
    qa.Tk = s.mode == FORWARD ? T : s.Tmax;
    qa.Hkv = Hkv; qa.rope = rope;
    GPT_TRY(mark(s, GPT_KERNEL_QKV, last, true));
    GPT_TRY(launch_qkv(dt, qa, s.st, sk));
    GPT_TRY(mark(s, GPT_KERNEL_QKV, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_ATTN, last, true));
    if (s.mode == STEP) {
      DecAttnArgs da{};
      da.q = q; da.k = kbuf; da.v = vbuf; da.kv_bh = kv_bh; da.Tmax = s.Tmax; da.pos = s.pos;
      da.o = o; da.o_ld = C; da.B = B; da.H = H; da.D = D; da.scale_log2 = scale_log2; da.Hkv = Hkv;
      da.alibi = alibi;
      GPT_TRY(launch_attention_decode(dt, da, s.st));
    } else {
      AttnArgs aa{};
      attn_headmajor(aa, q, (long long)T * D, kbuf, vbuf, kv_bh, H, Hkv, D);
      aa.o = o; aa.o_ld = C;
      aa.B = B; aa.H = H; aa.T_seq = T; aa.D = D; aa.Hkv = Hkv; aa.alibi = alibi;
      aa.scale_log2 = scale_log2;
      GPT_TRY(launch_attention(dt, aa, s.st));
    }
    GPT_TRY(mark(s, GPT_KERNEL_ATTN, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_PROJ, last, true));
    GPT_TRY(launch_linear_resid(dt, o, C, P.at(w.proj_w), C, nullptr, M, C, C, x, C, s.st, sk));
    GPT_TRY(mark(s, GPT_KERNEL_PROJ, last, false));
    la.g = P.at(w.ln2_g);
    GPT_TRY(mark(s, GPT_KERNEL_LN, last, true));
    GPT_TRY(launch_layernorm(dt, la, s.st));
    GPT_TRY(mark(s, GPT_KERNEL_LN, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_FC, last, true));
    GPT_TRY(launch_linear(dt, a, C, P.at(w.fc_w), C, nullptr, M, 2 * F, C, h, F, 3, 0, s.st, sk));
    GPT_TRY(mark(s, GPT_KERNEL_FC, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_FCPROJ, last, true));
    GPT_TRY(launch_linear_resid(dt, h, F, P.at(w.fcproj_w), F, nullptr, M, C, F, x, C, s.st, sk));
    GPT_TRY(mark(s, GPT_KERNEL_FCPROJ, last, false));
    if (l + 1 < L) {   // RMSNorm of the next block (the final one is applied by the caller)
      la.g = P.at(P.layer(l + 1).ln1_g);
      GPT_TRY(launch_layernorm(dt, la, s.st));
    }
  }
  return GPT_OK;
}

// Embedding and the L blocks; leaves the fp32 residual stream in ws.x (with
// no blocks, ws.a already holds ln_f of the embedding).
// Decode steps of bf16 pre-LN GPT-2 blocks split the K range of their three
// weight-streaming products into slices written as fp32 partial products
// (no block waits on another): the Q|K|U slices feed the decode attention,
// which finishes q, k, u and appends the cache row; the slices of c_proj and
// of mlp.c_proj feed a residual update fused with the LayerNorm that follows
// it (LN2, then LN1 of the next block or ln_f after the last one).  c_fc
// keeps its own GELU epilogue.  Slice counts: K / S a whole number of
// 64-deep stages from {2, 4, 6, 8, 12}, S M N within the partial buffer.
struct StepSplit { int qkv, proj, fcproj; };

static int pick_split(int K, int M, int N, size_t cap, const int* prefs, int n) {
  for (int i = 0; i < n; ++i) {
    const int S = prefs[i];
    if (K % S != 0) continue;
    const int d = K / S;
    if (d != 128 && d != 256 && d != 384 && d != 512 && d != 768) continue;
    if ((size_t)S * M * N <= cap) return S;
  }
  return 0;
}

bool step_split(const gpt_config* c, int M, const Plan& pl, StepSplit* sp) {
  if (c->dtype != GPT_BF16 || c->arch != 0 || c->post_ln != 0 || c->n_layer <= 0 || M > 64 || !pl.skpart)
    return false;
  const int C = c->n_embd, F = c->n_ff, D = C / c->n_head;
  if (C % 128 || F % 128 || D % 8 || C > 1024 || kv_heads(c) != c->n_head) return false;
  const size_t cap = (size_t)SK_PART_TILES * 64 * 32;
  static const int pq[] = {3, 6, 2, 4, 1}, pp[] = {6, 3, 4, 2, 1}, pf[] = {8, 12, 6, 4, 2, 1};
  StepSplit r{pick_split(C, M, 3 * C, cap, pq, 5), pick_split(C, M, C, cap, pp, 5), pick_split(F, M, C, cap, pf, 6)};
  if (!r.qkv || !r.proj || !r.fcproj) return false;
  if (sp) *sp = r;
  return true;
}

// The residual LayerNorms also read the weights of the two products that
// follow them (LN2: c_fc and mlp.c_proj; LN1: the next block's c_attn and
// c_proj) with blocks of their own, so those products find them cached.
static void prefetch(LnArgs& la, const void* w0, size_t b0, const void* w1, size_t b1) {
  la.pf[0] = w0; la.pf_bytes[0] = b0; la.pf_blocks[0] = w0 ? resid_ln_prefetch_blocks(b0) : 0;
  la.pf[1] = w1; la.pf_bytes[1] = b1; la.pf_blocks[1] = w1 ? resid_ln_prefetch_blocks(b1) : 0;
}

int run_blocks_step_split(const Pass& s, const StepSplit& sp) {
  const gpt_config* cfg = s.cfg;
  const Params& P = s.P;
  const int B = s.B, M = B, C = cfg->n_embd, F = cfg->n_ff;
  const int H = cfg->n_head, D = C / H, L = cfg->n_layer;
  float* x = at<float>(s.ws, s.pl.x);
  void* a = at<char>(s.ws, s.pl.a);
  void* o = at<char>(s.ws, s.pl.o);
  void* h = at<char>(s.ws, s.pl.h);
  float* part = at<float>(s.ws, s.pl.skpart);
  const size_t cap = (size_t)SK_PART_TILES * 64 * 32;
  const long long cache_layer = (long long)B * H * s.Tmax * D;
  SkinnyWs skw{part, SK_PART_TILES, at<int>(s.ws, s.pl.skcnt), SK_COUNTERS};

  LnArgs la{};
  la.M = M; la.C = C; la.T_seq = 1; la.eps = cfg->ln_eps;
  la.idx = s.idx; la.wte = P.at(0); la.wpe = P.at(P.wpe()); la.vocab = cfg->vocab; la.ctx = cfg->ctx;
  la.pos = s.pos;
  la.x = x; la.in_mul = 1; la.in_add = 0;
  la.g = P.at(P.layer(0).ln1_g); la.b = P.at(P.layer(0).ln1_b);
  la.out = a;
  la.zero = skw.cnt; la.zero_n = skw.cnt_len;   // counters of the other skinny products (c_fc uses none)
  GPT_TRY(launch_embed_ln(GPT_BF16, la, s.st));
  la.idx = nullptr; la.pos = nullptr; la.zero = nullptr; la.zero_n = 0;
  la.part = part;

  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  for (int l = 0; l < L; ++l) {
    const LayerP w = P.layer(l);
    const bool last = l == L - 1;
    GPT_TRY(mark(s, GPT_KERNEL_QKV, last, true));
    GPT_TRY(launch_skinny_slices(a, P.at(w.attn_w), M, 3 * C, C, sp.qkv, part, cap, s.st));
    GPT_TRY(mark(s, GPT_KERNEL_QKV, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_ATTN, last, true));
    DecAttnArgs da{};
    da.q = nullptr;
    da.k = static_cast<char*>(s.kc) + l * cache_layer * 2;
    da.v = static_cast<char*>(s.vc) + l * cache_layer * 2;
    da.kv_bh = (long long)s.Tmax * D; da.Tmax = s.Tmax; da.pos = s.pos;
    da.o = o; da.o_ld = C; da.B = B; da.H = H; da.D = D; da.scale_log2 = scale_log2; da.Hkv = H;
    GPT_TRY(launch_attention_decode_slices(da, part, sp.qkv, P.at(w.attn_b), s.st));
    GPT_TRY(mark(s, GPT_KERNEL_ATTN, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_PROJ, last, true));
    GPT_TRY(launch_skinny_slices(o, P.at(w.proj_w), M, C, C, sp.proj, part, cap, s.st));
    GPT_TRY(mark(s, GPT_KERNEL_PROJ, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_LN, last, true));
    la.nsplit = sp.proj; la.rbias = P.at(w.proj_b);
    la.g = P.at(w.ln2_g); la.b = P.at(w.ln2_b);
    prefetch(la, P.at(w.fc_w), (size_t)F * C * 2, P.at(w.fcproj_w), (size_t)C * F * 2);
    GPT_TRY(launch_resid_layernorm(la, s.st));
    GPT_TRY(mark(s, GPT_KERNEL_LN, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_FC, last, true));
    GPT_TRY(launch_linear(GPT_BF16, a, C, P.at(w.fc_w), C, P.at(w.fc_b), M, F, C, h, F, cfg->activation ? 2 : 1, 0,
                          s.st, &skw));
    GPT_TRY(mark(s, GPT_KERNEL_FC, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_FCPROJ, last, true));
    GPT_TRY(launch_skinny_slices(h, P.at(w.fcproj_w), M, C, F, sp.fcproj, part, cap, s.st));
    GPT_TRY(mark(s, GPT_KERNEL_FCPROJ, last, false));
    // ln_1 of the next block, or ln_f after the last one
    la.nsplit = sp.fcproj; la.rbias = P.at(w.fcproj_b);
    la.g = P.at(last ? P.lnf_g() : P.layer(l + 1).ln1_g);
    la.b = P.at(last ? P.lnf_b() : P.layer(l + 1).ln1_b);
    if (last) prefetch(la, nullptr, 0, nullptr, 0);
    else prefetch(la, P.at(P.layer(l + 1).attn_w), (size_t)3 * C * C * 2, P.at(P.layer(l + 1).proj_w), (size_t)C * C * 2);
    GPT_TRY(launch_resid_layernorm(la, s.st));
  }
  return GPT_OK;
}

int run_blocks(const Pass& s) {
  if (s.cfg->arch == 1) return run_blocks_llama(s);
  if (s.mode == STEP && !s.xs) {
    StepSplit sp;
    if (step_split(s.cfg, s.B, s.pl, &sp)) return run_blocks_step_split(s, sp);
  }
  const gpt_config* cfg = s.cfg;
  const Params& P = s.P;
  const int dt = cfg->dtype, B = s.B, T = s.T, M = B * T, C = cfg->n_embd, F = cfg->n_ff;
  const int H = cfg->n_head, D = C / H, L = cfg->n_layer;
  float* x = at<float>(s.ws, s.pl.x);
  void* a = at<char>(s.ws, s.pl.a);
  void* q = at<char>(s.ws, s.pl.q);
  void* o = at<char>(s.ws, s.pl.o);
  void* h = at<char>(s.ws, s.pl.h);
  const size_t es = esize(cfg);
  const long long cache_layer = (long long)B * H * s.Tmax * D;   // elements per layer of each cache
  SkinnyWs skw{};
  if (s.pl.skpart) skw = SkinnyWs{at<float>(s.ws, s.pl.skpart), SK_PART_TILES, at<int>(s.ws, s.pl.skcnt), SK_COUNTERS};
  const SkinnyWs* sk = s.pl.skpart ? &skw : nullptr;

  LnArgs la{};
  la.M = M; la.C = C; la.T_seq = T; la.eps = cfg->ln_eps;
  la.idx = s.idx; la.wte = P.at(0); la.wpe = P.at(P.wpe()); la.vocab = cfg->vocab; la.ctx = cfg->ctx;
  la.pos = s.mode == STEP ? s.pos : nullptr;
  la.x = x; la.in_mul = 1; la.in_add = 0;
  // pre-LN: the embedding kernel applies LN1 of block 0 (ln_f with no blocks);
  // post-LN: block 0 reads the embedding itself
  const bool post = cfg->post_ln != 0;
  la.ident = post ? 1 : 0;
  la.g = P.at(post ? 0 : (L > 0 ? P.layer(0).ln1_g : P.lnf_g()));
  la.b = P.at(post ? 0 : (L > 0 ? P.layer(0).ln1_b : P.lnf_b()));
  la.out = a;
  la.zero = sk ? skw.cnt : nullptr; la.zero_n = sk ? skw.cnt_len : 0;
  GPT_TRY(launch_embed_ln(dt, la, s.st));
  la.idx = nullptr; la.pos = nullptr; la.zero = nullptr; la.zero_n = 0; la.ident = 0;
  la.write_x = post ? 1 : 0;   // post-LN: each LayerNorm also replaces the residual row

  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  const size_t row_bytes = (size_t)M * C * sizeof(float);
  for (int l = 0; l < L; ++l) {
    const LayerP w = P.layer(l);
    const bool last = l == L - 1;
    if (s.xs) GPT_TRY(hipMemcpyAsync(s.xs + (size_t)l * M * C, x, row_bytes, hipMemcpyDeviceToDevice, s.st));
    void* kbuf = s.mode == FORWARD ? at<char>(s.ws, s.pl.k) : static_cast<char*>(s.kc) + l * cache_layer * es;
    void* vbuf = s.mode == FORWARD ? at<char>(s.ws, s.pl.v) : static_cast<char*>(s.vc) + l * cache_layer * es;
    const long long kv_bh = s.mode == FORWARD ? (long long)T * D : (long long)s.Tmax * D;
    // forward: c_attn writes token-major rows [M, 3C] (Q | K | U, head h at
    // columns h D of each third), which the attention reads in place; the
    // cache passes scatter K and U into the cache layout instead
    const bool rows = s.mode == FORWARD;
    GPT_TRY(mark(s, GPT_KERNEL_QKV, last, true));
    if (rows) {
      GPT_TRY(launch_linear(dt, a, C, P.at(w.attn_w), C, P.at(w.attn_b), M, 3 * C, C, q, 3 * C, 0, 0, s.st, sk));
    } else {
      QKVArgs qa{};
      qa.A = a; qa.W = P.at(w.attn_w); qa.bias = P.at(w.attn_b);
      qa.M = M; qa.C = C; qa.H = H; qa.D = D; qa.T_seq = T;
      qa.q = q; qa.q_bh = (long long)T * D;
      qa.k = kbuf; qa.k_bh = kv_bh;
      qa.v = vbuf; qa.v_bh = kv_bh;
      qa.pos = s.mode == STEP ? s.pos : nullptr;
      qa.Tk = s.Tmax;
      qa.Hkv = H; qa.rope = nullptr;
      GPT_TRY(launch_qkv(dt, qa, s.st, sk));
    }
    GPT_TRY(mark(s, GPT_KERNEL_QKV, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_ATTN, last, true));
    if (s.mode == STEP) {
      DecAttnArgs da{};
      da.q = q; da.k = kbuf; da.v = vbuf; da.kv_bh = kv_bh; da.Tmax = s.Tmax; da.pos = s.pos;
      da.o = o; da.o_ld = C; da.B = B; da.H = H; da.D = D; da.scale_log2 = scale_log2; da.Hkv = H;
      GPT_TRY(launch_attention_decode(dt, da, s.st));
    } else {
      AttnArgs aa{};
      if (rows) {
        const long long ld = 3LL * C;
        char* qkv = static_cast<char*>(q);
        aa.q = qkv;              aa.q_sb = T * ld; aa.q_sh = D; aa.q_st = (int)ld;
        aa.k = qkv + C * es;     aa.k_sb = T * ld; aa.k_sh = D; aa.k_st = (int)ld;
        aa.v = qkv + 2 * C * es; aa.v_sb = T * ld; aa.v_sh = D; aa.v_st = (int)ld;
      } else {
        attn_headmajor(aa, q, (long long)T * D, kbuf, vbuf, kv_bh, H, H, D);
      }
      aa.o = o; aa.o_ld = C;
      aa.B = B; aa.H = H; aa.T_seq = T; aa.D = D; aa.Hkv = H;
      aa.scale_log2 = scale_log2;
      GPT_TRY(launch_attention(dt, aa, s.st));
    }
    GPT_TRY(mark(s, GPT_KERNEL_ATTN, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_PROJ, last, true));
    GPT_TRY(launch_linear_resid(dt, o, C, P.at(w.proj_w), C, P.at(w.proj_b), M, C, C, x, C, s.st, sk));
    GPT_TRY(mark(s, GPT_KERNEL_PROJ, last, false));
    // pre-LN: a = LN2(x) feeds the MLP; post-LN: x = a = LN1(x + attn)
    la.g = P.at(post ? w.ln1_g : w.ln2_g); la.b = P.at(post ? w.ln1_b : w.ln2_b);
    GPT_TRY(mark(s, GPT_KERNEL_LN, last, true));
    GPT_TRY(launch_layernorm(dt, la, s.st));
    GPT_TRY(mark(s, GPT_KERNEL_LN, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_FC, last, true));
    GPT_TRY(launch_linear(dt, a, C, P.at(w.fc_w), C, P.at(w.fc_b), M, F, C, h, F, cfg->activation ? 2 : 1, 0, s.st,
                          sk));
    GPT_TRY(mark(s, GPT_KERNEL_FC, last, false));
    GPT_TRY(mark(s, GPT_KERNEL_FCPROJ, last, true));
    GPT_TRY(launch_linear_resid(dt, h, F, P.at(w.fcproj_w), F, P.at(w.fcproj_b), M, C, F, x, C, s.st, sk));
    GPT_TRY(mark(s, GPT_KERNEL_FCPROJ, last, false));
    if (post) {        // x = a = LN2(n + mlp(n)): the next block's input (or the final hidden)
      la.g = P.at(w.ln2_g); la.b = P.at(w.ln2_b);
      GPT_TRY(launch_layernorm(dt, la, s.st));
    } else if (l + 1 < L) {   // ln_1 of the next block (ln_f is applied by the caller)
      la.g = P.at(P.layer(l + 1).ln1_g); la.b = P.at(P.layer(l + 1).ln1_b);
      GPT_TRY(launch_layernorm(dt, la, s.st));
    }
  }
  if (s.xs) GPT_TRY(hipMemcpyAsync(s.xs + (size_t)L * M * C, x, row_bytes, hipMemcpyDeviceToDevice, s.st));
  return GPT_OK;
}

// ln_f of M rows: residual row (r * mul + add) -> dense row r of out.  With no
// blocks, the embedding kernel applied ln_f already (to every row, into ws.a);
// post-LN models have no ln_f and ws.a holds the final hidden rows.
bool rows_final(const gpt_config* c) { return c->n_layer == 0 || c->post_ln != 0; }

int final_norm(const Pass& s, int M, int mul, int add, void* out) {
  const gpt_config* cfg = s.cfg;
  LnArgs la{};
  la.M = M; la.C = cfg->n_embd; la.T_seq = s.T; la.eps = cfg->ln_eps;
  la.x = at<float>(s.ws, s.pl.x); la.in_mul = mul; la.in_add = add;
  la.g = s.P.at(s.P.lnf_g()); la.b = s.P.opt(s.P.lnf_b());
  la.rms = cfg->arch == 1 ? 1 : 0;   // LLaMA-style: the final RMSNorm
  la.out = out;
  return hip_status(launch_layernorm(cfg->dtype, la, s.st));
}

int check_cache_args(const gpt_config* cfg, void* kc, void* vc, int Tmax, int B) {
  if (!kc || !vc) return GPT_ERR_NULL;
  if (Tmax <= 0 || Tmax > cfg->ctx || Tmax > 4096 || B <= 0) return GPT_ERR_SHAPE;
  return GPT_OK;
}

// Workspace of the head backward.  dz [M, Vp] and its transpose [V, Np], the
// head matrix's transpose [C, Vp] and a's [C, Np] are zero-padded along the
// contracted axis (Vp to a multiple of 256, Np of 64), so both gradient
// products run without a K tail.  The vocabulary contraction of da = dz W
// (a small [M, C] output) is split into S slices of Vp / S (fp32 partials,
// summed in slice order) so that its tiles fill the CUs.
struct BwdPlan {
  size_t a, aT, ET, dz, dzT, pmax, psum, tgt, tok, bsum, lse, yv, inv, da, dapart, mu, rs, lnpart, total;
  int ntiles, nblocks, Vp, Np, nchunks, S;
};

// Slices of the vocabulary contraction: the S in {1, 2, 4, 8} with the least
// time per slice-round (rounds of blocks over the CUs, divided by S), the
// smallest on a tie; Vp / S stays a whole number of stages and at least 256.
static int da_split(int dtype, size_t M, size_t C, int Vp) {
  if (dtype == 0) return 1;
  // C a multiple of 192: 128 x 192 tiles, two blocks per CU (512 per round);
  // otherwise 256 x 256 tiles, one per CU
  const bool t192 = C % 192 == 0;
  const long long tiles = t192 ? (long long)((M + 127) / 128) * (long long)(C / 192)
                               : (long long)((M + 255) / 256) * (long long)((C + 255) / 256);
  const long long round = t192 ? 512 : 256;
  const int quantum = t192 ? 64 : 32;
  int best = 1;
  double best_t = (double)((tiles + round - 1) / round);
  for (int S = 2; S <= 8; S *= 2) {
    if (Vp % S != 0 || (Vp / S) % quantum != 0 || Vp / S < 256) break;
    const double t = (double)((tiles * S + round - 1) / round) / S;
    if (t < best_t) { best_t = t; best = S; }
  }
  return best;
}

constexpr long long BWD_MAX_ROWS = 1LL << 20;

BwdPlan bwd_plan(const gpt_config* c, int B, int T) {
  BwdPlan p{};
  const size_t M = (size_t)B * T, C = c->n_embd, V = c->vocab, es = esize(c);
  p.ntiles = head_ntiles(c->dtype, (int)M, c->vocab, c->n_embd, false);
  p.nblocks = ce_reduce_blocks((int)M);
  p.Vp = (int)align_up(V, 256);
  p.Np = (int)align_up(M, 64);
  p.S = da_split(c->dtype, M, C, p.Vp);
  p.nchunks = ln_bwd_chunks((int)M);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  p.a = take(M * C * es);
  p.aT = take(C * p.Np * es);
  p.ET = take(C * p.Vp * es);
  p.dz = take(M * p.Vp * es);
  p.dzT = take(V * p.Np * es);
  p.pmax = take(M * p.ntiles * 4);
  p.psum = take(M * p.ntiles * 4);
  p.tgt = take(M * 4);
  p.tok = take(M * 4);
  p.bsum = take((size_t)p.nblocks * 2 * 8);
  p.lse = take(M * 4);
  p.yv = take(M * 4);
  p.inv = take(4);
  p.da = take(M * C * 4);
  p.dapart = take(p.S > 1 ? (size_t)p.S * M * C * 4 : 0);
  p.mu = take(M * 4);
  p.rs = take(M * 4);
  p.lnpart = take((size_t)p.nchunks * 2 * C * 4);
  p.total = off;
  return p;
}

// Workspace of one block's backward (pre-LN GPT-2 blocks): the recomputed
// forward (a1, q, k, u, o, x1, a2, u_fc, h), the compute-dtype copies and
// zero-padded transposes the gradient products read ([rows, Mp] with Mp = M
// rounded up to 64, and the four weight transposes), and the fp32 gradients
// of the intermediate tensors.
constexpr int DW_SPLIT = 4;

struct BlkPlan {
  size_t a1, q, k, v, o, x1, a2, uf, hm, dyc, dyT, hT, dh, duc, duT, a2T, da, dx1, dx1c, dx1T, oT, dout, dqkv,
      dqkvc, dqkvT, a1T, aS, aP, aPT, adS, adST, adoc, adOT, aKT, aQT, alse, aDv, wfpT, wfcT, wpT, waT, mu, rs, part,
      wpart, total;
  int Mp, Fp, C3p, Tp, nchunks;
};

BlkPlan blk_plan(const gpt_config* c, int B, int T) {
  BlkPlan p{};
  const size_t M = (size_t)B * T, C = c->n_embd, F = c->n_ff, es = esize(c), H = c->n_head;
  p.Mp = (int)align_up(M, 64);
  p.Fp = (int)align_up(F, 64);
  p.C3p = (int)align_up(3 * C, 64);
  p.nchunks = ln_bwd_chunks((int)M);
  const size_t Mp = p.Mp;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  p.a1 = take(M * C * es); p.q = take(M * C * es); p.k = take(M * C * es); p.v = take(M * C * es);
  p.o = take(M * C * es); p.x1 = take(M * C * 4); p.a2 = take(M * C * es); p.uf = take(M * F * es);
  p.hm = take(M * F * es); p.dyc = take(M * C * es); p.dyT = take(C * Mp * es); p.hT = take(F * Mp * es);
  p.dh = take(M * F * 4); p.duc = take(M * F * es); p.duT = take(F * Mp * es); p.a2T = take(C * Mp * es);
  p.da = take(M * C * 4); p.dx1 = take(M * C * 4); p.dx1c = take(M * C * es); p.dx1T = take(C * Mp * es);
  p.oT = take(C * Mp * es); p.dout = take(M * C * 4); p.dqkv = take(M * 3 * C * 4); p.dqkvc = take(M * 3 * C * es);
  p.dqkvT = take(3 * C * Mp * es); p.a1T = take(C * Mp * es);
  // attention backward: per-head score matrices [B*H][T][Tp] and transposes [B*H][D][Tp]
  p.Tp = (int)align_up((size_t)T, 64);
  const size_t Z = (size_t)B * H, TT = (size_t)T * p.Tp, DT = (C / H) * (size_t)p.Tp;
  // (S / dP and the row-major P are stored only by the fp32 path: the bf16
  // one fuses them away)
  p.aS = take(c->dtype == 0 ? Z * TT * 4 : 0); p.aP = take(c->dtype == 0 ? Z * TT * es : 0); p.aPT = take(Z * TT * es); p.adS = take(Z * TT * es);
  p.adST = take(Z * TT * es); p.adoc = take(M * C * es); p.adOT = take(Z * DT * es); p.aKT = take(Z * DT * es);
  p.aQT = take(Z * DT * es);
  p.alse = take(Z * T * 4); p.aDv = take(Z * T * 4);   // per-row log-sum-exp (log2) and dO . O
  p.wfpT = take(F * C * es); p.wfcT = take(C * (size_t)p.Fp * es); p.wpT = take(C * C * es);
  p.waT = take(C * (size_t)p.C3p * es);
  p.mu = take(M * 4); p.rs = take(M * 4);
  // column partials: the widest of the sums (3C for the c_attn bias, F for c_fc's, 2C for a LayerNorm)
  const size_t nch = std::max<size_t>(p.nchunks, colsum_chunks((int)M));
  p.part = take(nch * (3 * C > F ? 3 * C : F) * 4);
  // split-K partials of the weight gradients: room for DW_SPLIT copies of the largest [3C, C] or [F, C]
  p.wpart = take((size_t)DW_SPLIT * C * (3 * C > F ? 3 * C : F) * 4);
  p.total = off;
  return p;
}

int decode_step_impl(const gpt_config* cfg, const void* params, const int32_t* tok, int B, int32_t* pos,
                     void* k_cache, void* v_cache, int Tmax, int32_t* next_tok, void* logits, void* ws,
                     size_t ws_bytes, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!params || !tok || !ws || !pos || !next_tok) return GPT_ERR_NULL;
  s = check_cache_args(cfg, k_cache, v_cache, Tmax, B);
  if (s != GPT_OK) return s;
  const Plan pl = plan(cfg, B, 1, true);
  if (ws_bytes < pl.total) return GPT_ERR_WORKSPACE;

  Pass ps{cfg, params_of(cfg, params), tok, B, 1, STEP, pos, k_cache, v_cache, Tmax, ws, pl,
          static_cast<hipStream_t>(stream), nullptr, nullptr, -1};
  s = run_blocks(ps);
  if (s != GPT_OK) return s;
  void* a = at<char>(ws, pl.a);
  if (!rows_final(cfg) && !step_split(cfg, B, pl, nullptr)) {   // the split step applied ln_f already
    s = final_norm(ps, B, 1, 0, a);
    if (s != GPT_OK) return s;
  }
  const int V = cfg->vocab;
  GPT_TRY(launch_head_ce(cfg->dtype, a, ps.P.at(ps.P.head_w()), B, V, cfg->n_embd, logits, V,
                         at<float>(ws, pl.pmax), nullptr, nullptr, at<int32_t>(ws, pl.pidx), nullptr, nullptr, 1,
                         ps.st));
  GPT_TRY(launch_argmax_reduce(B, pl.ntiles, at<float>(ws, pl.pmax), at<int32_t>(ws, pl.pidx), next_tok, pos, -1,
                               ps.st));
  return GPT_OK;
}

// Scratch of gpt_decode_step_noalloc (for callers that cannot allocate): one
// copy of this array per GPU, held until the process ends.  Host code never
// uses the array's name as an address: the device address is fetched once per
// device with hipGetSymbolAddress (that device current) and kept per device.
static __device__ __align__(256) char scratch[GPT_DECODE_NOALLOC_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The current device's copy of `scratch`.
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  if (g_scratch_ptr[dev] == nullptr) return hipErrorInvalidSymbol;
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int64_t gpt_param_count(const gpt_config* cfg) {
  const int s = check_config(cfg);
  if (s != GPT_OK) return s;
  return offsets(cfg, nullptr, 0);
}

int gpt_param_offsets(const gpt_config* cfg, int64_t* off, int n) {
  const int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!off) return GPT_ERR_NULL;
  if (n < offset_count(cfg)) return GPT_ERR_SHAPE;
  offsets(cfg, off, n);
  return GPT_OK;
}

int gpt_workspace_bytes(const gpt_config* cfg, int B, int T, size_t* bytes) {
  const int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!bytes) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0) return GPT_ERR_SHAPE;
  if (T > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  *bytes = plan(cfg, B, T, false).total;
  return GPT_OK;
}

int gpt_decode_workspace_bytes(const gpt_config* cfg, int B, int Tp, size_t* bytes) {
  const int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!bytes) return GPT_ERR_NULL;
  if (B <= 0 || Tp <= 0) return GPT_ERR_SHAPE;
  if (Tp > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  const size_t pre = plan(cfg, B, Tp, true).total, step = plan(cfg, B, 1, true).total;
  *bytes = pre > step ? pre : step;   // one workspace serves the prefill and every step
  return GPT_OK;
}

const char* gpt_status_string(int status) {
  switch (status) {
    case GPT_OK: return "ok";
    case GPT_ERR_NULL: return "a required pointer is NULL";
    case GPT_ERR_CONFIG: return "invalid model configuration (dims, C % H, alignment of C, n_ff or D, D > 128)";
    case GPT_ERR_SEQ_TOO_LONG: return "sequence length T exceeds the context length";
    case GPT_ERR_SHAPE: return "invalid shape argument";
    case GPT_ERR_WORKSPACE: return "workspace too small";
    case GPT_ERR_DTYPE: return "unsupported dtype";
    case GPT_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    default: return "unknown status";
  }
}

int gpt_forward(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                const int32_t* targets, void* logits, float* token_loss, float* mean_loss, void* ws,
                size_t ws_bytes, void* stream) {
  return gpt_forward_timed(cfg, params, idx, B, T, targets, logits, 0, token_loss, mean_loss, ws, ws_bytes, stream,
                           nullptr, nullptr, -1);
}

int gpt_forward_ld(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                   const int32_t* targets, void* logits, long long ld_logits, float* token_loss, float* mean_loss,
                   void* ws, size_t ws_bytes, void* stream) {
  return gpt_forward_timed(cfg, params, idx, B, T, targets, logits, ld_logits, token_loss, mean_loss, ws, ws_bytes,
                           stream, nullptr, nullptr, -1);
}

int gpt_forward_timed(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                      const int32_t* targets, void* logits, long long ld_logits, float* token_loss,
                      float* mean_loss, void* ws, size_t ws_bytes, void* stream, void* ev_begin, void* ev_end,
                      int which) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!params || !idx || !ws) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0) return GPT_ERR_SHAPE;
  if (ld_logits == 0) ld_logits = cfg->vocab;
  if (ld_logits < cfg->vocab || ld_logits > (1LL << 31)) return GPT_ERR_SHAPE;
  if (T > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  if ((long long)B * T > (1LL << 24)) return GPT_ERR_SHAPE;
  const Plan pl = plan(cfg, B, T, false);
  if (ws_bytes < pl.total) return GPT_ERR_WORKSPACE;

  Pass ps{cfg, params_of(cfg, params), idx, B, T, FORWARD, nullptr, nullptr, nullptr, T, ws, pl,
          static_cast<hipStream_t>(stream), ev_begin, ev_end, which};
  s = run_blocks(ps);
  if (s != GPT_OK) return s;
  const int M = B * T, V = cfg->vocab, C = cfg->n_embd;
  void* a = at<char>(ws, pl.a);
  if (!rows_final(cfg)) {
    s = final_norm(ps, M, 1, 0, a);
    if (s != GPT_OK) return s;
  }
  float* tok = token_loss ? token_loss : at<float>(ws, pl.tok);
  GPT_TRY(mark(ps, GPT_KERNEL_HEAD, true, true));
  GPT_TRY(launch_head_ce(cfg->dtype, a, ps.P.at(ps.P.head_w()), M, V, C, logits, ld_logits, at<float>(ws, pl.pmax),
                         at<float>(ws, pl.psum), at<float>(ws, pl.tgt), nullptr, targets, idx, T, ps.st));
  GPT_TRY(mark(ps, GPT_KERNEL_HEAD, true, false));
  GPT_TRY(launch_ce_reduce(M, pl.ntiles, at<float>(ws, pl.pmax), at<float>(ws, pl.psum), at<float>(ws, pl.tgt),
                           targets, idx, T, V, tok, at<double>(ws, pl.bsum), mean_loss, ps.st));
  return GPT_OK;
}

int gpt_prefill(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int Tp, void* k_cache,
                void* v_cache, int Tmax, int32_t* pos, int32_t* next_tok, void* last_logits, void* ws,
                size_t ws_bytes, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!params || !idx || !ws || !pos || !next_tok) return GPT_ERR_NULL;
  s = check_cache_args(cfg, k_cache, v_cache, Tmax, B);
  if (s != GPT_OK) return s;
  if (Tp <= 0) return GPT_ERR_SHAPE;
  if (Tp > Tmax) return GPT_ERR_SEQ_TOO_LONG;
  if ((long long)B * Tp > (1LL << 24)) return GPT_ERR_SHAPE;
  const Plan pl = plan(cfg, B, Tp, true);
  if (ws_bytes < pl.total) return GPT_ERR_WORKSPACE;

  Pass ps{cfg, params_of(cfg, params), idx, B, Tp, PREFILL, nullptr, k_cache, v_cache, Tmax, ws, pl,
          static_cast<hipStream_t>(stream), nullptr, nullptr, -1};
  s = run_blocks(ps);
  if (s != GPT_OK) return s;
  // the greedy choice uses the last position of every sequence only
  void* alast = at<char>(ws, pl.alast);
  s = !rows_final(cfg) ? final_norm(ps, B, Tp, Tp - 1, alast) : GPT_OK;
  if (s != GPT_OK) return s;
  if (rows_final(cfg))   // rows of ws.a already hold the final hidden: gather the last ones
    GPT_TRY(hipMemcpy2DAsync(alast, esize(cfg) * cfg->n_embd, at<char>(ws, pl.a) + (size_t)(Tp - 1) * esize(cfg) * cfg->n_embd,
                             (size_t)Tp * esize(cfg) * cfg->n_embd, esize(cfg) * cfg->n_embd, B, hipMemcpyDeviceToDevice,
                             ps.st));
  const int V = cfg->vocab;
  GPT_TRY(launch_head_ce(cfg->dtype, alast, ps.P.at(ps.P.head_w()), B, V, cfg->n_embd, last_logits, V,
                         at<float>(ws, pl.pmax), nullptr, nullptr, at<int32_t>(ws, pl.pidx), nullptr, nullptr, 1,
                         ps.st));
  GPT_TRY(launch_argmax_reduce(B, pl.ntiles, at<float>(ws, pl.pmax), at<int32_t>(ws, pl.pidx), next_tok, pos, Tp,
                               ps.st));
  return GPT_OK;
}

int gpt_decode_step(const gpt_config* cfg, const void* params, const int32_t* tok, int B, int32_t* pos,
                    void* k_cache, void* v_cache, int Tmax, int32_t* next_tok, void* logits, void* ws,
                    size_t ws_bytes, void* stream) {
  return decode_step_impl(cfg, params, tok, B, pos, k_cache, v_cache, Tmax, next_tok, logits, ws, ws_bytes, stream);
}

int gpt_decode_step_noalloc(const gpt_config* cfg, const void* params, const int32_t* tok, int B, int32_t* pos,
                            void* k_cache, void* v_cache, int Tmax, int32_t* next_tok, void* logits, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!params || !tok || !pos || !next_tok) return GPT_ERR_NULL;
  s = check_cache_args(cfg, k_cache, v_cache, Tmax, B);
  if (s != GPT_OK) return s;
  if (plan(cfg, B, 1, true).total > (size_t)GPT_DECODE_NOALLOC_BYTES) return GPT_ERR_WORKSPACE;
  void* ws = nullptr;
  GPT_TRY(noalloc_scratch(&ws));
  return decode_step_impl(cfg, params, tok, B, pos, k_cache, v_cache, Tmax, next_tok, logits, ws,
                          (size_t)GPT_DECODE_NOALLOC_BYTES, stream);
}

int gpt_sample(const gpt_config* cfg, const void* logits, int B, const gpt_sampling* sp, const float* u,
               uint32_t* seen, int32_t* next_tok, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!logits || !sp || !next_tok) return GPT_ERR_NULL;
  if (B <= 0) return GPT_ERR_SHAPE;
  if (cfg->vocab > 53248) return GPT_ERR_CONFIG;
  if (!std::isfinite(sp->temperature) || !(sp->top_p > 0.f) || !std::isfinite(sp->top_p) ||
      !(sp->repetition_penalty > 0.f) || !std::isfinite(sp->repetition_penalty))
    return GPT_ERR_SHAPE;
  if (sp->temperature > 0.f && !u) return GPT_ERR_NULL;
  SampleArgs a{};
  a.logits = logits; a.ld = cfg->vocab; a.V = cfg->vocab; a.B = B;
  a.temperature = sp->temperature; a.top_k = sp->top_k; a.top_p = sp->top_p; a.penalty = sp->repetition_penalty;
  a.u = u; a.seen = seen; a.seen_words = (cfg->vocab + 31) / 32; a.out = next_tok;
  return hip_status(launch_sample(cfg->dtype, a, static_cast<hipStream_t>(stream)));
}

int gpt_mark_seen(const gpt_config* cfg, const int32_t* tokens, int B, int T, uint32_t* seen, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!tokens || !seen) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0) return GPT_ERR_SHAPE;
  return hip_status(launch_mark_seen(tokens, B, T, cfg->vocab, seen, static_cast<hipStream_t>(stream)));
}

int gpt_head_backward_workspace_bytes(const gpt_config* cfg, int B, int T, size_t* bytes) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (cfg->arch != 0) return GPT_ERR_CONFIG;
  if (!bytes) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0 || (long long)B * T > BWD_MAX_ROWS) return GPT_ERR_SHAPE;
  if (T > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  *bytes = bwd_plan(cfg, B, T).total;
  return GPT_OK;
}

int gpt_head_backward(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                      const int32_t* targets, const float* x, float* dx, float* grads, float* mean_loss, void* ws,
                      size_t ws_bytes, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (cfg->arch != 0) return GPT_ERR_CONFIG;   // the final RMSNorm's backward is not provided
  if (!params || !idx || !x || !dx || !grads || !ws) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0 || (long long)B * T > BWD_MAX_ROWS) return GPT_ERR_SHAPE;
  if (T > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  const BwdPlan pl = bwd_plan(cfg, B, T);
  if (ws_bytes < pl.total) return GPT_ERR_WORKSPACE;
  const Params P = params_of(cfg, params);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = cfg->dtype, M = B * T, V = cfg->vocab, C = cfg->n_embd;
  const bool post = cfg->post_ln != 0;
  const void* Wh = P.at(P.head_w());
  void* a = at<char>(ws, pl.a);

  // final hidden rows in the compute dtype: ln_f(x), or x itself (post-LN)
  if (!post) {
    LnArgs la{};
    la.M = M; la.C = C; la.T_seq = T; la.eps = cfg->ln_eps;
    la.x = const_cast<float*>(x); la.in_mul = 1; la.in_add = 0;   // read only (write_x is 0)
    la.g = P.at(P.lnf_g()); la.b = P.at(P.lnf_b());
    la.out = a;
    GPT_TRY(launch_layernorm(dt, la, st));
  } else {
    GPT_TRY(launch_cast_rows(dt, x, (long long)M * C, a, st));
  }
  // log-sum-exp of every row, targets, 1 / n_valid and the mean loss
  GPT_TRY(launch_head_ce(dt, a, Wh, M, V, C, nullptr, 0, at<float>(ws, pl.pmax), at<float>(ws, pl.psum),
                         at<float>(ws, pl.tgt), nullptr, targets, idx, T, st));
  GPT_TRY(launch_ce_reduce(M, pl.ntiles, at<float>(ws, pl.pmax), at<float>(ws, pl.psum), at<float>(ws, pl.tgt),
                           targets, idx, T, V, at<float>(ws, pl.tok), at<double>(ws, pl.bsum), mean_loss, st));
  GPT_TRY(launch_bwd_rows(M, pl.ntiles, at<float>(ws, pl.pmax), at<float>(ws, pl.psum), targets, idx, T, V,
                          at<float>(ws, pl.lse), at<int32_t>(ws, pl.yv), at<float>(ws, pl.inv), st));
  // dz = (softmax - onehot) / n_valid, recomputed from the fp32 accumulators of a second head product
  // (written in both layouts: dz [M, Vp] and dzT [V, Np]; the pads are zeroed)
  void* dz = at<char>(ws, pl.dz);
  void* dzT = at<char>(ws, pl.dzT);
  GPT_TRY(launch_head_dz(dt, a, Wh, M, V, C, at<float>(ws, pl.lse), at<int32_t>(ws, pl.yv), at<float>(ws, pl.inv),
                         dz, pl.Vp, dzT, pl.Np, st));
  GPT_TRY(launch_zero_cols(dt, dz, pl.Vp, M, V, pl.Vp, st));
  GPT_TRY(launch_zero_cols(dt, dzT, pl.Np, V, M, pl.Np, st));
  void* ET = at<char>(ws, pl.ET);
  void* aT = at<char>(ws, pl.aT);
  GPT_TRY(launch_transpose(dt, Wh, C, V, C, ET, pl.Vp, st));
  GPT_TRY(launch_transpose(dt, a, C, M, C, aT, pl.Np, st));
  // da = dz W_head (contraction over the padded vocabulary); post-LN: that is dx
  float* da = post ? dx : at<float>(ws, pl.da);
  if (pl.S > 1) {
    GPT_TRY(launch_gemm_f32_splitk(dt, dz, pl.Vp, ET, pl.Vp, M, C, pl.Vp / pl.S, pl.S, at<float>(ws, pl.dapart),
                                   (long long)M * C, st));
    GPT_TRY(launch_add_partials(da, at<float>(ws, pl.dapart), (long long)M * C, pl.S, st, 0));
  } else {
    GPT_TRY(launch_gemm_f32out(dt, dz, pl.Vp, ET, pl.Vp, M, C, pl.Vp, da, C, 0, st));
  }
  // dW_head += dz^T a (contraction over the padded rows)
  GPT_TRY(launch_gemm_f32out(dt, dzT, pl.Np, aT, pl.Np, V, C, pl.Np, grads + P.head_w(), C, 1, st));
  if (!post)
    GPT_TRY(launch_ln_backward(dt, M, C, x, P.at(P.lnf_g()), da, cfg->ln_eps, dx, at<float>(ws, pl.mu),
                               at<float>(ws, pl.rs), at<float>(ws, pl.lnpart), grads + P.lnf_g(), grads + P.lnf_b(),
                               st, 0));
  return GPT_OK;
}

int gpt_embedding_backward(const gpt_config* cfg, const int32_t* idx, int B, int T, const float* dx0, float* grads,
                           void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!idx || !dx0 || !grads) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0 || (long long)B * T > (1LL << 24)) return GPT_ERR_SHAPE;
  if (T > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  const int64_t wpe = params_of(cfg, nullptr).wpe();   // LLaMA-style models have no position table
  GPT_TRY(launch_embed_backward(idx, B, T, cfg->n_embd, cfg->vocab, dx0, grads, wpe < 0 ? nullptr : grads + wpe,
                                static_cast<hipStream_t>(stream)));
  return GPT_OK;
}

int gpt_forward_train(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                      const int32_t* targets, float* xs, float* mean_loss, void* ws, size_t ws_bytes, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (cfg->arch != 0 || cfg->post_ln != 0) return GPT_ERR_CONFIG;   // pre-LN GPT-2 blocks only
  if (!params || !idx || !xs || !ws) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0) return GPT_ERR_SHAPE;
  if (T > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  if ((long long)B * T > BWD_MAX_ROWS) return GPT_ERR_SHAPE;
  const Plan pl = plan(cfg, B, T, false);
  if (ws_bytes < pl.total) return GPT_ERR_WORKSPACE;
  Pass ps{cfg, params_of(cfg, params), idx, B, T, FORWARD, nullptr, nullptr, nullptr, T, ws, pl,
          static_cast<hipStream_t>(stream), nullptr, nullptr, -1, xs};
  s = run_blocks(ps);
  if (s != GPT_OK) return s;
  if (!mean_loss) return GPT_OK;   // only the residual streams (the head backward computes the loss again)
  const int M = B * T, V = cfg->vocab, C = cfg->n_embd;
  void* a = at<char>(ws, pl.a);
  if (!rows_final(cfg)) {
    s = final_norm(ps, M, 1, 0, a);
    if (s != GPT_OK) return s;
  }
  GPT_TRY(launch_head_ce(cfg->dtype, a, ps.P.at(ps.P.head_w()), M, V, C, nullptr, V, at<float>(ws, pl.pmax),
                         at<float>(ws, pl.psum), at<float>(ws, pl.tgt), nullptr, targets, idx, T, ps.st));
  GPT_TRY(launch_ce_reduce(M, pl.ntiles, at<float>(ws, pl.pmax), at<float>(ws, pl.psum), at<float>(ws, pl.tgt),
                           targets, idx, T, V, at<float>(ws, pl.tok), at<double>(ws, pl.bsum), mean_loss, ps.st));
  return GPT_OK;
}

int gpt_block_backward_workspace_bytes(const gpt_config* cfg, int B, int T, size_t* bytes) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (cfg->arch != 0 || cfg->post_ln != 0) return GPT_ERR_CONFIG;
  if (!bytes) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0 || (long long)B * T > BWD_MAX_ROWS) return GPT_ERR_SHAPE;
  if (T > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  *bytes = blk_plan(cfg, B, T).total;
  return GPT_OK;
}

int gpt_block_backward(const gpt_config* cfg, const void* params, int layer, int B, int T, const float* x,
                       const float* dy, float* dx, float* grads, void* ws, size_t ws_bytes, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (cfg->arch != 0 || cfg->post_ln != 0) return GPT_ERR_CONFIG;
  if (!params || !x || !dy || !dx || !grads || !ws) return GPT_ERR_NULL;
  if (layer < 0 || layer >= cfg->n_layer) return GPT_ERR_SHAPE;
  if (B <= 0 || T <= 0 || (long long)B * T > BWD_MAX_ROWS) return GPT_ERR_SHAPE;
  if (T > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  const BlkPlan pl = blk_plan(cfg, B, T);
  if (ws_bytes < pl.total) return GPT_ERR_WORKSPACE;
  const Params P = params_of(cfg, params);
  const LayerP w = P.layer(layer);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = cfg->dtype, M = B * T, C = cfg->n_embd, F = cfg->n_ff, H = cfg->n_head, D = C / H;
  const int Mp = pl.Mp, act = cfg->activation;
  const size_t rowf = (size_t)M * C * 4;
  auto W = [&](size_t off) { return at<char>(ws, off); };
  auto Wf = [&](size_t off) { return at<float>(ws, off); };
  // weight gradient out [R, N] += A [R, Mp] . B [N, Mp]^T (contraction over the
  // padded tokens): split into S slices of Mp run as one launch into fp32
  // partials, then added in slice order (deterministic).  S doubles until
  // about 256 output tiles of 128 x 192 are in flight (at most 16 slices,
  // within the partials buffer).
  auto dW = [&](const void* A, const void* Bm, int R, int N, float* out) -> hipError_t {
    const long long tiles = (long long)((R + 127) / 128) * ((N + 191) / 192);
    const long long cap = (long long)DW_SPLIT * C * (3 * C > F ? 3 * C : F);
    int S = 1;
    while (S < 16 && tiles * S < 256 && Mp % (64 * 2 * S) == 0 && 2LL * S * R * N <= cap) S *= 2;
    const int Ks = Mp / S;
    const hipError_t e = launch_gemm_f32_splitk(dt, A, Mp, Bm, Mp, R, N, Ks, S, Wf(pl.wpart), (long long)R * N, st);
    if (e != hipSuccess) return e;
    return launch_add_partials(out, Wf(pl.wpart), (long long)R * N, S, st);
  };

  // ---- recompute the block's forward from its input x
  LnArgs la{};
  la.M = M; la.C = C; la.T_seq = T; la.eps = cfg->ln_eps; la.in_mul = 1; la.in_add = 0;
  la.x = const_cast<float*>(x); la.g = P.at(w.ln1_g); la.b = P.at(w.ln1_b); la.out = W(pl.a1);   // read only
  GPT_TRY(launch_layernorm(dt, la, st));
  QKVArgs qa{};
  qa.A = W(pl.a1); qa.W = P.at(w.attn_w); qa.bias = P.at(w.attn_b);
  qa.M = M; qa.C = C; qa.H = H; qa.D = D; qa.T_seq = T;
  qa.q = W(pl.q); qa.q_bh = (long long)T * D; qa.k = W(pl.k); qa.k_bh = (long long)T * D;
  qa.v = W(pl.v); qa.v_bh = (long long)T * D; qa.pos = nullptr; qa.Tk = T; qa.Hkv = H; qa.rope = nullptr;
  GPT_TRY(launch_qkv(dt, qa, st, nullptr));
  AttnArgs aa{};
  attn_headmajor(aa, W(pl.q), (long long)T * D, W(pl.k), W(pl.v), (long long)T * D, H, H, D);
  aa.o = W(pl.o); aa.o_ld = C;
  aa.B = B; aa.H = H; aa.T_seq = T; aa.D = D; aa.Hkv = H;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  aa.lse2 = Wf(pl.alse);
  GPT_TRY(launch_attention(dt, aa, st));
  float* x1 = Wf(pl.x1);
  GPT_TRY(hipMemcpyAsync(x1, x, rowf, hipMemcpyDeviceToDevice, st));
  GPT_TRY(launch_linear_resid(dt, W(pl.o), C, P.at(w.proj_w), C, P.at(w.proj_b), M, C, C, x1, C, st, nullptr));
  la.x = x1; la.g = P.at(w.ln2_g); la.b = P.at(w.ln2_b); la.out = W(pl.a2);
  GPT_TRY(launch_layernorm(dt, la, st));
  GPT_TRY(launch_linear(dt, W(pl.a2), C, P.at(w.fc_w), C, P.at(w.fc_b), M, F, C, W(pl.uf), F, 0, 0, st, nullptr));
  GPT_TRY(launch_act_fwd(dt, W(pl.uf), (long long)M * F, act, W(pl.hm), st));

  // ---- weight transposes (operands with the contraction axis contiguous)
  GPT_TRY(launch_transpose(dt, P.at(w.fcproj_w), F, C, F, W(pl.wfpT), C, st));    // [C,F] -> [F,C]
  GPT_TRY(launch_transpose(dt, P.at(w.fc_w), C, F, C, W(pl.wfcT), pl.Fp, st));    // [F,C] -> [C,Fp]
  GPT_TRY(launch_transpose(dt, P.at(w.proj_w), C, C, C, W(pl.wpT), C, st));      // [C,C] -> [C,C]
  GPT_TRY(launch_transpose(dt, P.at(w.attn_w), C, 3 * C, C, W(pl.waT), pl.C3p, st));   // [3C,C] -> [C,3Cp]

  // ---- MLP: dh = dy Wfp, dWfp += dy^T h, dbfp += sum dy
  GPT_TRY(launch_cast_transpose(dt, dy, M, C, W(pl.dyc), W(pl.dyT), Mp, st));
  GPT_TRY(launch_gemm_f32out(dt, W(pl.dyc), C, W(pl.wfpT), C, M, F, C, Wf(pl.dh), F, 0, st));
  GPT_TRY(launch_transpose(dt, W(pl.hm), F, M, F, W(pl.hT), Mp, st));
  GPT_TRY(dW(W(pl.dyT), W(pl.hT), C, F, grads + w.fcproj_w));
  GPT_TRY(launch_colsum(M, C, dy, Wf(pl.part), grads + w.fcproj_b, st));
  // du = dh * GELU'(u); dWfc += du^T a2; dbfc += sum du; da2 = du Wfc
  GPT_TRY(launch_act_bwd(dt, Wf(pl.dh), W(pl.uf), (long long)M * F, act, W(pl.duc), st));
  GPT_TRY(launch_colsum(M, F, Wf(pl.dh), Wf(pl.part), grads + w.fc_b, st));
  GPT_TRY(launch_transpose(dt, W(pl.duc), F, M, F, W(pl.duT), Mp, st));
  GPT_TRY(launch_transpose(dt, W(pl.a2), C, M, C, W(pl.a2T), Mp, st));
  GPT_TRY(dW(W(pl.duT), W(pl.a2T), F, C, grads + w.fc_w));
  GPT_TRY(launch_gemm_f32out(dt, W(pl.duc), F, W(pl.wfcT), pl.Fp, M, C, F, Wf(pl.da), C, 0, st));
  // dx1 = dy + LN2 backward
  float* dx1 = Wf(pl.dx1);
  GPT_TRY(hipMemcpyAsync(dx1, dy, rowf, hipMemcpyDeviceToDevice, st));
  GPT_TRY(launch_ln_backward(dt, M, C, x1, P.at(w.ln2_g), Wf(pl.da), cfg->ln_eps, dx1, Wf(pl.mu), Wf(pl.rs),
                             Wf(pl.part), grads + w.ln2_g, grads + w.ln2_b, st, 1));

  // ---- attention: dWp += dx1^T o, dbp += sum dx1, dO = dx1 Wp
  GPT_TRY(launch_cast_transpose(dt, dx1, M, C, W(pl.dx1c), W(pl.dx1T), Mp, st));
  GPT_TRY(launch_transpose(dt, W(pl.o), C, M, C, W(pl.oT), Mp, st));
  GPT_TRY(dW(W(pl.dx1T), W(pl.oT), C, C, grads + w.proj_w));
  GPT_TRY(launch_colsum(M, C, dx1, Wf(pl.part), grads + w.proj_b, st));
  GPT_TRY(launch_gemm_f32out(dt, W(pl.dx1c), C, W(pl.wpT), C, M, C, C, Wf(pl.dout), C, 0, st));
  const AttnBwdWs aw{Wf(pl.aS), W(pl.aP), W(pl.aPT), W(pl.adS), W(pl.adST), W(pl.adoc), W(pl.adOT), W(pl.aKT),
                     W(pl.aQT), pl.Tp, Wf(pl.alse), W(pl.o), Wf(pl.aDv)};
  GPT_TRY(launch_attention_backward(dt, W(pl.q), W(pl.k), W(pl.v), Wf(pl.dout), Wf(pl.dqkv), B, H, T, D, aw, st));
  // dWattn += dqkv^T a1, dbattn += sum dqkv, da1 = dqkv Wattn
  GPT_TRY(launch_colsum(M, 3 * C, Wf(pl.dqkv), Wf(pl.part), grads + w.attn_b, st));
  GPT_TRY(launch_cast_transpose(dt, Wf(pl.dqkv), M, 3 * C, W(pl.dqkvc), W(pl.dqkvT), Mp, st));
  GPT_TRY(launch_transpose(dt, W(pl.a1), C, M, C, W(pl.a1T), Mp, st));
  GPT_TRY(dW(W(pl.dqkvT), W(pl.a1T), 3 * C, C, grads + w.attn_w));
  GPT_TRY(launch_gemm_f32out(dt, W(pl.dqkvc), 3 * C, W(pl.waT), pl.C3p, M, C, 3 * C, Wf(pl.da), C, 0, st));
  // dx = dx1 + LN1 backward
  GPT_TRY(hipMemcpyAsync(dx, dx1, rowf, hipMemcpyDeviceToDevice, st));
  GPT_TRY(launch_ln_backward(dt, M, C, x, P.at(w.ln1_g), Wf(pl.da), cfg->ln_eps, dx, Wf(pl.mu), Wf(pl.rs),
                             Wf(pl.part), grads + w.ln1_g, grads + w.ln1_b, st, 1));
  return GPT_OK;
}

int gpt_debug_layernorm(const gpt_config* cfg, const float* x, const void* g, const void* b, int M, void* out,
                        void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!x || !g || !b || !out) return GPT_ERR_NULL;
  if (M <= 0) return GPT_ERR_SHAPE;
  LnArgs la{};
  la.M = M; la.C = cfg->n_embd; la.T_seq = 1; la.eps = cfg->ln_eps;
  la.x = const_cast<float*>(x); la.in_mul = 1; la.in_add = 0;
  la.g = g; la.b = b; la.out = out;
  return hip_status(launch_layernorm(cfg->dtype, la, static_cast<hipStream_t>(stream)));
}

int gpt_debug_linear(const gpt_config* cfg, const void* A, const void* W, const void* bias, int M, int N, int K,
                     int act, int out_f32, void* out, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!A || !W || !out) return GPT_ERR_NULL;
  if (M <= 0 || N <= 0 || K <= 0 || K % vec_of(cfg) != 0 || act < 0 || act > 2) return GPT_ERR_SHAPE;
  return hip_status(launch_linear(cfg->dtype, A, K, W, K, bias, M, N, K, out, N, act, out_f32 ? 1 : 0,
                                  static_cast<hipStream_t>(stream)));
}

int gpt_debug_attention(const gpt_config* cfg, const void* q, const void* k, const void* u, int B, int T,
                        void* out, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!q || !k || !u || !out) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0) return GPT_ERR_SHAPE;
  const int C = cfg->n_embd, H = cfg->n_head, D = C / H;
  AttnArgs aa{};
  attn_headmajor(aa, q, (long long)T * D, k, u, (long long)T * D, cfg->n_head, cfg->n_head, cfg->n_embd / cfg->n_head);
  aa.o = out; aa.o_ld = C;
  aa.B = B; aa.H = H; aa.T_seq = T; aa.D = D; aa.Hkv = H;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  return hip_status(launch_attention(cfg->dtype, aa, static_cast<hipStream_t>(stream)));
}

int gpt_debug_attention_rows(const gpt_config* cfg, const void* qkv, int B, int T, void* out, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!qkv || !out) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0) return GPT_ERR_SHAPE;
  const int C = cfg->n_embd, H = cfg->n_head, D = C / H;
  const long long ld = 3LL * C;
  const size_t es = cfg->dtype == 0 ? 4 : 2;
  const char* rows = static_cast<const char*>(qkv);
  AttnArgs aa{};
  aa.q = rows;              aa.q_sb = T * ld; aa.q_sh = D; aa.q_st = (int)ld;
  aa.k = rows + C * es;     aa.k_sb = T * ld; aa.k_sh = D; aa.k_st = (int)ld;
  aa.v = rows + 2 * C * es; aa.v_sb = T * ld; aa.v_sh = D; aa.v_st = (int)ld;
  aa.o = out; aa.o_ld = C;
  aa.B = B; aa.H = H; aa.T_seq = T; aa.D = D; aa.Hkv = H;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  return hip_status(launch_attention(cfg->dtype, aa, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
