// Host side of the C ABI declared in include/gptmi.h: validation, parameter
// blob offsets, workspace plan and the launch sequence of the forward pass.
// Stateless: every call validates on the host, then enqueues kernels on the
// caller's stream and returns without synchronising.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../include/gptmi.h"
#include "kernels.h"

using namespace gptmi;

namespace {

thread_local char g_hip_msg[256] = "";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return GPT_OK;
  snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return GPT_ERR_HIP;
}

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
  if (c->n_embd % c->n_head != 0) return GPT_ERR_CONFIG;
  const int D = c->n_embd / c->n_head, v = vec_of(c);
  if (c->n_embd % v || c->n_ff % v || D % v || D > 128 || c->n_embd > 2048) return GPT_ERR_CONFIG;
  return GPT_OK;
}

// Parameter blob views (element offsets), packing order as documented.
struct LayerP { int64_t ln1_g, ln1_b, attn_w, attn_b, proj_w, proj_b, ln2_g, ln2_b, fc_w, fc_b, fcproj_w, fcproj_b; };

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
  put(ctx * C);
  for (int l = 0; l < c->n_layer; ++l) {
    put(C); put(C); put(3 * C * C); put(3 * C); put(C * C); put(C);
    put(C); put(C); put(F * C); put(F); put(C * F); put(C);
  }
  put(C);
  put(C);
  if (out && k < n) out[k] = off;
  return off;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Plan {
  size_t x, a, q, k, v, o, h, pmax, psum, tgt, tok, bsum, total;
  int ntiles, nblocks;
};

Plan plan(const gpt_config* c, int B, int T) {
  Plan p{};
  const size_t M = (size_t)B * T, C = c->n_embd, F = c->n_ff, es = esize(c);
  p.ntiles = (c->vocab + head_tile_n(c->dtype) - 1) / head_tile_n(c->dtype);
  p.nblocks = ce_reduce_blocks((int)M);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  p.x = take(M * C * 4);
  p.a = take(M * C * es);
  p.q = take(M * C * es);
  p.k = take(M * C * es);
  p.v = take(M * C * es);
  p.o = take(M * C * es);
  p.h = take(M * F * es);
  p.pmax = take(M * p.ntiles * 4);
  p.psum = take(M * p.ntiles * 4);
  p.tgt = take(M * 4);
  p.tok = take(M * 4);
  p.bsum = take((size_t)p.nblocks * 2 * 8);
  p.total = off;
  return p;
}

template <typename P> P* at(void* base, size_t off) { return reinterpret_cast<P*>(static_cast<char*>(base) + off); }

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
  if (n < 2 + 12 * cfg->n_layer + 3) return GPT_ERR_SHAPE;
  offsets(cfg, off, n);
  return GPT_OK;
}

int gpt_workspace_bytes(const gpt_config* cfg, int B, int T, size_t* bytes) {
  const int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!bytes) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0) return GPT_ERR_SHAPE;
  if (T > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  *bytes = plan(cfg, B, T).total;
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
    case GPT_ERR_HIP: return g_hip_msg[0] ? g_hip_msg : "HIP error";
    default: return "unknown status";
  }
}

int gpt_forward(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                const int32_t* targets, void* logits, float* token_loss, float* mean_loss, void* ws,
                size_t ws_bytes, void* stream) {
  return gpt_forward_timed(cfg, params, idx, B, T, targets, logits, token_loss, mean_loss, ws, ws_bytes, stream,
                           nullptr, nullptr, -1);
}

int gpt_forward_timed(const gpt_config* cfg, const void* params, const int32_t* idx, int B, int T,
                      const int32_t* targets, void* logits, float* token_loss, float* mean_loss, void* ws,
                      size_t ws_bytes, void* stream, void* ev_begin, void* ev_end, int which) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!params || !idx || !ws) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0) return GPT_ERR_SHAPE;
  if (T > cfg->ctx) return GPT_ERR_SEQ_TOO_LONG;
  if ((long long)B * T > (1LL << 30)) return GPT_ERR_SHAPE;
  const Plan p = plan(cfg, B, T);
  if (ws_bytes < p.total) return GPT_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  // Records the caller's events around one launch (timing hook; no-op by default).
  auto mark = [&](int kind, bool last_layer, bool begin) -> hipError_t {
    if (kind != which || !last_layer) return hipSuccess;
    void* ev = begin ? ev_begin : ev_end;
    return ev ? hipEventRecord(static_cast<hipEvent_t>(ev), st) : hipSuccess;
  };
  const int dt = cfg->dtype, M = B * T, C = cfg->n_embd, F = cfg->n_ff, H = cfg->n_head, D = C / H;
  const int L = cfg->n_layer, V = cfg->vocab;
  const float eps = cfg->ln_eps;
  const size_t es = esize(cfg);
  const char* P = static_cast<const char*>(params);
  auto poff = [&](int64_t e) { return static_cast<const void*>(P + e * (int64_t)es); };
  const int64_t V_C = (int64_t)V * C, ctxC = (int64_t)cfg->ctx * C;
  const int64_t per_layer = 4 * (int64_t)C * C + 4 * C + 2 * (int64_t)C * F + F + C + 4 * C;
  auto layer_base = [&](int l) { return V_C + ctxC + (int64_t)l * per_layer; };
  auto lp = [&](int l) {
    const int64_t b = layer_base(l);
    LayerP r;
    r.ln1_g = b;
    r.ln1_b = r.ln1_g + C;
    r.attn_w = r.ln1_b + C;
    r.attn_b = r.attn_w + 3LL * C * C;
    r.proj_w = r.attn_b + 3LL * C;
    r.proj_b = r.proj_w + (int64_t)C * C;
    r.ln2_g = r.proj_b + C;
    r.ln2_b = r.ln2_g + C;
    r.fc_w = r.ln2_b + C;
    r.fc_b = r.fc_w + (int64_t)F * C;
    r.fcproj_w = r.fc_b + F;
    r.fcproj_b = r.fcproj_w + (int64_t)C * F;
    return r;
  };
  const int64_t lnf_g = layer_base(L), lnf_b = lnf_g + C;

  float* x = at<float>(ws, p.x);
  void* a = at<char>(ws, p.a);
  void* q = at<char>(ws, p.q);
  void* k = at<char>(ws, p.k);
  void* v = at<char>(ws, p.v);
  void* o = at<char>(ws, p.o);
  void* h = at<char>(ws, p.h);
  float* pmax = at<float>(ws, p.pmax);
  float* psum = at<float>(ws, p.psum);
  float* tgt = at<float>(ws, p.tgt);
  float* tok = token_loss ? token_loss : at<float>(ws, p.tok);
  double* bsum = at<double>(ws, p.bsum);

  {
    const int64_t g0 = L > 0 ? lp(0).ln1_g : lnf_g, b0 = L > 0 ? lp(0).ln1_b : lnf_b;
    GPT_TRY(launch_embed_ln(dt, M, C, T, eps, idx, poff(0), poff(V_C), V, x, poff(g0), poff(b0), a, st));
  }
  AttnArgs aa{};
  aa.q = q; aa.q_bh = (long long)T * D;
  aa.k = k; aa.k_bh = (long long)T * D;
  aa.v = v; aa.v_bh = (long long)T * D;
  aa.o = o; aa.o_ld = C;
  aa.B = B; aa.H = H; aa.T_seq = T; aa.D = D;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  for (int l = 0; l < L; ++l) {
    const LayerP w = lp(l);
    QKVArgs qa{};
    qa.A = a; qa.W = poff(w.attn_w); qa.bias = poff(w.attn_b);
    qa.M = M; qa.C = C; qa.H = H; qa.D = D; qa.T_seq = T;
    qa.q = q; qa.q_bh = (long long)T * D;
    qa.k = k; qa.k_bh = (long long)T * D;
    qa.v = v; qa.v_bh = (long long)T * D;
    qa.pos = nullptr;
    const bool last = l == L - 1;
    GPT_TRY(mark(GPT_KERNEL_QKV, last, true));
    GPT_TRY(launch_qkv(dt, qa, st));
    GPT_TRY(mark(GPT_KERNEL_QKV, last, false));
    GPT_TRY(mark(GPT_KERNEL_ATTN, last, true));
    GPT_TRY(launch_attention(dt, aa, st));
    GPT_TRY(mark(GPT_KERNEL_ATTN, last, false));
    GPT_TRY(mark(GPT_KERNEL_PROJ, last, true));
    GPT_TRY(launch_linear_resid(dt, o, C, poff(w.proj_w), C, poff(w.proj_b), M, C, C, x, C, st));
    GPT_TRY(mark(GPT_KERNEL_PROJ, last, false));
    GPT_TRY(mark(GPT_KERNEL_LN, last, true));
    GPT_TRY(launch_layernorm(dt, M, C, eps, x, poff(w.ln2_g), poff(w.ln2_b), a, st));
    GPT_TRY(mark(GPT_KERNEL_LN, last, false));
    GPT_TRY(mark(GPT_KERNEL_FC, last, true));
    GPT_TRY(launch_linear(dt, a, C, poff(w.fc_w), C, poff(w.fc_b), M, F, C, h, F, 1, 0, st));
    GPT_TRY(mark(GPT_KERNEL_FC, last, false));
    GPT_TRY(mark(GPT_KERNEL_FCPROJ, last, true));
    GPT_TRY(launch_linear_resid(dt, h, F, poff(w.fcproj_w), F, poff(w.fcproj_b), M, C, F, x, C, st));
    GPT_TRY(mark(GPT_KERNEL_FCPROJ, last, false));
    const int64_t ng = l + 1 < L ? lp(l + 1).ln1_g : lnf_g, nb = l + 1 < L ? lp(l + 1).ln1_b : lnf_b;
    GPT_TRY(launch_layernorm(dt, M, C, eps, x, poff(ng), poff(nb), a, st));
  }
  GPT_TRY(mark(GPT_KERNEL_HEAD, true, true));
  GPT_TRY(launch_head_ce(dt, a, poff(0), M, V, C, logits, V, pmax, psum, tgt, targets, idx, T, st));
  GPT_TRY(mark(GPT_KERNEL_HEAD, true, false));
  GPT_TRY(launch_ce_reduce(M, p.ntiles, pmax, psum, tgt, targets, idx, T, V, tok, bsum, mean_loss, st));
  return GPT_OK;
}

int gpt_debug_layernorm(const gpt_config* cfg, const float* x, const void* g, const void* b, int M, void* out,
                        void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!x || !g || !b || !out) return GPT_ERR_NULL;
  if (M <= 0) return GPT_ERR_SHAPE;
  return hip_status(launch_layernorm(cfg->dtype, M, cfg->n_embd, cfg->ln_eps, x, g, b, out,
                                     static_cast<hipStream_t>(stream)));
}

int gpt_debug_linear(const gpt_config* cfg, const void* A, const void* W, const void* bias, int M, int N, int K,
                     int act, int out_f32, void* out, void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!A || !W || !out) return GPT_ERR_NULL;
  if (M <= 0 || N <= 0 || K <= 0 || K % vec_of(cfg) != 0 || (act != 0 && act != 1)) return GPT_ERR_SHAPE;
  return hip_status(launch_linear(cfg->dtype, A, K, W, K, bias, M, N, K, out, N, act, out_f32 ? 1 : 0,
                                  static_cast<hipStream_t>(stream)));
}

int gpt_debug_attention(const gpt_config* cfg, const void* q, const void* k, const void* u, int B, int T, void* out,
                        void* stream) {
  int s = check_config(cfg);
  if (s != GPT_OK) return s;
  if (!q || !k || !u || !out) return GPT_ERR_NULL;
  if (B <= 0 || T <= 0) return GPT_ERR_SHAPE;
  const int C = cfg->n_embd, H = cfg->n_head, D = C / H;
  AttnArgs aa{};
  aa.q = q; aa.q_bh = (long long)T * D;
  aa.k = k; aa.k_bh = (long long)T * D;
  aa.v = u; aa.v_bh = (long long)T * D;
  aa.o = out; aa.o_ld = C;
  aa.B = B; aa.H = H; aa.T_seq = T; aa.D = D;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  return hip_status(launch_attention(cfg->dtype, aa, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
