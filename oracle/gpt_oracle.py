"""fp64 CPU oracle of the GPT-2-style decoder-only forward pass, loss and greedy decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may use it.  It shares no code with the HIP library; its only inputs are
plain numpy arrays (parameters upcast exactly to float64, int token ids).

Every function is the plain definition written out in float64 numpy, step by
step in the order the pages give, with no blocking, fusion or reordering.
Sources (web pages, cited by title and section):

  [P1] "预训练一个 Mini GPT（1.24 亿参数）" (ai-engineering.com.cn lesson):
       概念 / 注意力 / KV cache; 构建它 第1步..第7步.
  [P2] "第 25 章 从小 GPT 到 GPT-2：先把模型对上，再谈训练" (book.ozine.me): §25.1-§25.7.
  [P3] "Day 16: 从零组装 MiniGPT——第一次写出完整 GPT 模型" (yeyulingfeng.com).
  [P4] "02 GPT 架构——Decoder-Only 的自回归语言模型" (ting.is-a.dev).
  [P5] "GPT-1学习笔记：“预训练+微调”范式" (cs-knowledge-wiki): §3.2, §3.4, §3.6, §4.1, §6.1.

Readings where the pages are silent or disagree (pre-norm, tanh GELU, biases on
c_attn/c_proj, -inf mask, eps inside the square root with biased variance,
1/sqrt(D) scale, target shift, lowest-index argmax) are listed with the pins
that check them in the project's design notes.

Parity status: every function below is pinned by a CPU test against a closed
form, an identity, a brute-force computation, a library routine or a printed
value of the pages; the full-model numeric values themselves are not printed
by any page, so beyond those pins and the causal / batch / cache invariants
the end-to-end logits are "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# Parameter count, [P2] §25.4: per block 12C^2+13C (attention 4C^2+4C, MLP
# 8C^2+5C, two LayerNorms 4C); plus VC token table, ctx*C position table and
# the final LayerNorm's 2C.  The tied head adds nothing.  With an explicit
# MLP width F the per-block term is 4C^2+4C + 2CF+F+C + 4C.
# ----------------------------------------------------------------------------
def param_count(vocab: int, n_embd: int, n_layer: int, ctx: int, n_ff: Optional[int] = None,
                post_ln: bool = False, untied: bool = False) -> int:
    """post_ln: GPT-1 blocks with no final LayerNorm ([P5] §4.1 feeds the last
    block's output to the head); untied: a separate V x C head matrix without
    bias ([P3] 二十三 LM Head)."""
    C = n_embd
    F = 4 * C if n_ff is None else n_ff
    per_block = (4 * C * C + 4 * C) + (2 * C * F + F + C) + 4 * C
    return n_layer * per_block + vocab * C + ctx * C + (0 if post_ln else 2 * C) + (vocab * C if untied else 0)


# ----------------------------------------------------------------------------
# Building blocks
# ----------------------------------------------------------------------------
def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the last axis: g*(x-mean)/sqrt(var+eps)+b, biased variance,
    eps inside the square root ([P1] 第4步 LayerNorm; [P5] §3.2)."""
    mean = x.mean(axis=-1, keepdims=True)
    centred = x - mean
    var = (centred * centred).mean(axis=-1, keepdims=True)
    return g * centred / np.sqrt(var + eps) + b


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))
    ([P5] §3.6 激活函数; [P2] §25.3 keeps the approximation)."""
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def gelu_erf(z: np.ndarray) -> np.ndarray:
    """GELU, exact form: z Phi(z) = 0.5 z (1 + erf(z / sqrt(2))) ([P5] §3.6 标准公式;
    [P3] builds the MLP with nn.GELU(), whose default is this form)."""
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def activation(z: np.ndarray, act: str = "tanh") -> np.ndarray:
    return gelu_erf(z) if act == "erf" else gelu_tanh(z)


def linear(x: np.ndarray, W: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """y = x W^T + b with W stored [out, in] ([P2] §25.5: a Linear stores
    C_out x C_in and computes X W^T)."""
    y = x @ W.T
    if b is not None:
        y = y + b
    return y


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, subtracting the row maximum first
    ([P1] 第2步: softmax(x - c) = softmax(x))."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def causal_attention(q: np.ndarray, k: np.ndarray, u: np.ndarray) -> np.ndarray:
    """One head: A = softmax(q k^T / sqrt(D) + M), y = A u, with M[t,s] = -inf for
    s > t ([P2] §25.2: M is -inf where s>t; the value tensor is written U there;
    [P1] 注意力 divides by sqrt(d_k)).  q, k, u: [T, D]."""
    T, D = q.shape
    s = (q @ k.T) / math.sqrt(D)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    s = np.where(mask, -np.inf, s)
    return softmax_rows(s) @ u


def brute_attention(q: np.ndarray, k: np.ndarray, u: np.ndarray) -> np.ndarray:
    """The same head computed with explicit loops over (t, s <= t, d); tiny inputs only."""
    T, D = q.shape
    y = np.zeros((T, u.shape[1]))
    for t in range(T):
        scores = []
        for s in range(t + 1):
            acc = 0.0
            for d in range(D):
                acc += q[t, d] * k[s, d]
            scores.append(acc / math.sqrt(D))
        mx = max(scores)
        w = [math.exp(v - mx) for v in scores]
        tot = sum(w)
        for s in range(t + 1):
            for j in range(u.shape[1]):
                y[t, j] += (w[s] / tot) * u[s, j]
    return y


# ----------------------------------------------------------------------------
# The model
# ----------------------------------------------------------------------------
def embed(params: dict, idx: np.ndarray) -> np.ndarray:
    """x[b,t] = E[idx[b,t]] + P[t] ([P2] §25.1; [P1] 第1步; [P5] §4.1 h0 = U W_e + W_p)."""
    idx = np.asarray(idx)
    V = params["wte"].shape[0]
    if idx.min() < 0 or idx.max() >= V:
        raise ValueError("token id outside [0, V)")
    T = idx.shape[-1]
    if T > params["wpe"].shape[0]:
        raise ValueError("sequence longer than the context length")
    return params["wte"][idx] + params["wpe"][:T]


def attention_sublayer(a: np.ndarray, lp: dict, n_head: int, trace: Optional[dict] = None) -> np.ndarray:
    """Fused c_attn projection, split into Q|K|U along the last axis, heads as
    column blocks [hD,(h+1)D), per-head causal attention, heads merged back and
    c_proj applied ([P2] §25.2; [P5] §3.4 c_attn)."""
    B, T, C = a.shape
    D = C // n_head
    qkv = linear(a, lp["attn_w"], lp["attn_b"])                      # [B,T,3C]
    q, k, u = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]       # [B,T,C] each
    qh = q.reshape(B, T, n_head, D).transpose(0, 2, 1, 3)            # [B,H,T,D]
    kh = k.reshape(B, T, n_head, D).transpose(0, 2, 1, 3)
    uh = u.reshape(B, T, n_head, D).transpose(0, 2, 1, 3)
    y = np.empty_like(qh)
    for b in range(B):
        for h in range(n_head):
            y[b, h] = causal_attention(qh[b, h], kh[b, h], uh[b, h])
    o = y.transpose(0, 2, 1, 3).reshape(B, T, C)
    if trace is not None:
        trace.setdefault("c_attn", qkv.shape)
        trace.setdefault("split", q.shape)
        trace.setdefault("heads", qh.shape)
        trace.setdefault("scores", (B, n_head, T, T))
        trace.setdefault("merged", o.shape)
    return linear(o, lp["proj_w"], lp["proj_b"])


def mlp_sublayer(a: np.ndarray, lp: dict, act: str = "tanh") -> np.ndarray:
    """C -> F -> C with GELU in between ([P2] §25.3; tanh form unless act="erf")."""
    return linear(activation(linear(a, lp["fc_w"], lp["fc_b"]), act), lp["fcproj_w"], lp["fcproj_b"])


def block(x: np.ndarray, lp: dict, n_head: int, eps: float, trace: Optional[dict] = None,
          act: str = "tanh") -> np.ndarray:
    """Pre-norm block: x += attn(LN1(x)); x += mlp(LN2(x)) ([P1] Transformer 块 and
    第4步; [P2] §25.1; [P5] §3.2 notes GPT-2's move to pre-LN)."""
    x = x + attention_sublayer(layer_norm(x, lp["ln1_g"], lp["ln1_b"], eps), lp, n_head, trace)
    x = x + mlp_sublayer(layer_norm(x, lp["ln2_g"], lp["ln2_b"], eps), lp, act)
    return x


def block_post(x: np.ndarray, lp: dict, n_head: int, eps: float, act: str = "tanh") -> np.ndarray:
    """Post-norm (GPT-1) block: n = LN1(x + attn(x)); h = LN2(n + mlp(n))
    ([P5] §3.1 Block.forward, §3.2 Post-LN)."""
    n = layer_norm(x + attention_sublayer(x, lp, n_head), lp["ln1_g"], lp["ln1_b"], eps)
    return layer_norm(n + mlp_sublayer(n, lp, act), lp["ln2_g"], lp["ln2_b"], eps)


def final_hidden(params: dict, idx: np.ndarray, n_head: int, eps: float = 1e-5,
                 trace: Optional[dict] = None) -> np.ndarray:
    """ln_f(blocks(embed(idx))) -> [B,T,C]; for post-LN models the last block's
    output itself ([P5] §4.1: the head reads h_n)."""
    act = params.get("act", "tanh")
    x = embed(params, idx)
    if params.get("norm", "pre") == "post":
        for lp in params["layers"]:
            x = block_post(x, lp, n_head, eps, act)
        return x
    for lp in params["layers"]:
        x = block(x, lp, n_head, eps, trace, act)
    return layer_norm(x, params["lnf_g"], params["lnf_b"], eps)


def head(params: dict, a: np.ndarray) -> np.ndarray:
    """Tied head: logits = a E^T with the same E as the token lookup ([P2] §25.4;
    [P1] 第5步 logits = x @ token_embed.T; [P5] §4.1 softmax(h_n W_e^T)); with an
    untied head, a W_head^T ([P3] 二十三: nn.Linear(C, V, bias=False))."""
    return a @ params.get("head_w", params["wte"]).T


def derived_targets(idx: np.ndarray) -> np.ndarray:
    """Next-token targets from the inputs themselves: y[b,t] = idx[b,t+1] for
    t < T-1, and no target (-1) for the last position ([P2] §25.7: predict the
    next token, shift once only)."""
    idx = np.asarray(idx)
    y = np.full(idx.shape, -1, dtype=np.int64)
    y[:, :-1] = idx[:, 1:]
    return y


def cross_entropy_rows(z: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Per-row loss logsumexp(z) - z[y], computed as max + log sum exp(z - max)
    ([P1] 第6步 cross_entropy_loss).  Rows with y < 0 get 0."""
    m = z.max(axis=-1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=-1))
    rows = np.arange(z.shape[0])
    yy = np.where(y >= 0, y, 0)
    loss = lse - z[rows, yy]
    return np.where(y >= 0, loss, 0.0)


def forward(params: dict, idx: np.ndarray, n_head: int, eps: float = 1e-5,
            targets: Optional[np.ndarray] = None, want_logits: bool = True,
            row_chunk: int = 256, trace: Optional[dict] = None
            ) -> Tuple[Optional[np.ndarray], np.ndarray, float]:
    """Full forward + next-token cross-entropy.

    targets None: derived targets (shift by one, last position ignored);
    otherwise explicit [B,T] targets with -1 = ignore.  Returns
    (logits [B,T,V] fp64 or None, per-token loss [B,T] with 0 where ignored,
    mean loss over the positions that have a target).  The head and the loss
    are evaluated in row chunks only to bound memory; each row is the same
    computation.
    """
    idx = np.asarray(idx)
    B, T = idx.shape
    a = final_hidden(params, idx, n_head, eps, trace)
    y = derived_targets(idx) if targets is None else np.asarray(targets, dtype=np.int64)
    V = params.get("head_w", params["wte"]).shape[0]
    if y.max() >= V:
        raise ValueError("target outside [0, V)")
    a2 = a.reshape(B * T, -1)
    y2 = y.reshape(B * T)
    logits = np.empty((B * T, V)) if want_logits else None
    tok = np.empty(B * T)
    for r0 in range(0, B * T, row_chunk):
        z = head(params, a2[r0:r0 + row_chunk])
        tok[r0:r0 + row_chunk] = cross_entropy_rows(z, y2[r0:r0 + row_chunk])
        if want_logits:
            logits[r0:r0 + row_chunk] = z
    valid = y2 >= 0
    mean = float(tok[valid].sum() / valid.sum()) if valid.any() else float("nan")
    if want_logits:
        logits = logits.reshape(B, T, V)
    return logits, tok.reshape(B, T), mean


def argmax_lowest(z: np.ndarray) -> np.ndarray:
    """Greedy choice over the last axis; the lowest index wins ties ([P5] §6.1
    greedy generation takes the argmax of the last position's logits)."""
    return np.argmax(z, axis=-1)


# ----------------------------------------------------------------------------
# Greedy decode ([P1] 第7步 and KV cache; [P5] §6.1): two independent
# formulations that must agree.
# ----------------------------------------------------------------------------
def greedy_recompute(params: dict, prompt: np.ndarray, steps: int, n_head: int, eps: float = 1e-5):
    """Re-run the whole forward over the growing sequence for every new token and
    take the argmax of the last position.  Returns (tokens [B, steps+1],
    last-position logits [B, steps+1, V])."""
    seq = np.asarray(prompt).copy()
    toks, zs = [], []
    for _ in range(steps + 1):
        a = final_hidden(params, seq, n_head, eps)[:, -1]
        z = head(params, a)
        nxt = argmax_lowest(z)
        toks.append(nxt)
        zs.append(z)
        seq = np.concatenate([seq, nxt[:, None].astype(seq.dtype)], axis=1)
    return np.stack(toks, 1)[:, :steps + 1], np.stack(zs, 1)


def greedy_cached(params: dict, prompt: np.ndarray, steps: int, n_head: int, eps: float = 1e-5,
                  forced: Optional[np.ndarray] = None):
    """Prefill the prompt while storing every layer's per-head K and U, then for
    each step compute q/k/u of the new token only, append k/u to the cache and
    attend over all cached positions ([P1] KV cache).  With `forced` [B, steps]
    the fed tokens are taken from it (teacher forcing) instead of the argmax.
    Returns (emitted tokens [B, steps+1], last-position logits [B, steps+1, V])."""
    prompt = np.asarray(prompt)
    B, T0 = prompt.shape
    L = len(params["layers"])
    C = params["wte"].shape[1]
    D = C // n_head
    kc = [None] * L  # each [B,H,t,D]
    uc = [None] * L

    post = params.get("norm", "pre") == "post"
    act = params.get("act", "tanh")

    def run(tokens: np.ndarray, pos0: int) -> np.ndarray:
        n = tokens.shape[1]
        x = params["wte"][tokens] + params["wpe"][pos0:pos0 + n]
        for l, lp in enumerate(params["layers"]):
            a = x if post else layer_norm(x, lp["ln1_g"], lp["ln1_b"], eps)
            qkv = linear(a, lp["attn_w"], lp["attn_b"])
            q = qkv[..., :C].reshape(B, n, n_head, D).transpose(0, 2, 1, 3)
            k = qkv[..., C:2 * C].reshape(B, n, n_head, D).transpose(0, 2, 1, 3)
            u = qkv[..., 2 * C:].reshape(B, n, n_head, D).transpose(0, 2, 1, 3)
            kc[l] = k if kc[l] is None else np.concatenate([kc[l], k], axis=2)
            uc[l] = u if uc[l] is None else np.concatenate([uc[l], u], axis=2)
            tot = kc[l].shape[2]
            y = np.empty_like(q)
            for b in range(B):
                for h in range(n_head):
                    s = q[b, h] @ kc[l][b, h].T / math.sqrt(D)            # [n, tot]
                    qpos = pos0 + np.arange(n)[:, None]
                    s = np.where(np.arange(tot)[None, :] > qpos, -np.inf, s)
                    y[b, h] = softmax_rows(s) @ uc[l][b, h]
            o = y.transpose(0, 2, 1, 3).reshape(B, n, C)
            if post:
                x = layer_norm(x + linear(o, lp["proj_w"], lp["proj_b"]), lp["ln1_g"], lp["ln1_b"], eps)
                x = layer_norm(x + mlp_sublayer(x, lp, act), lp["ln2_g"], lp["ln2_b"], eps)
            else:
                x = x + linear(o, lp["proj_w"], lp["proj_b"])
                x = x + mlp_sublayer(layer_norm(x, lp["ln2_g"], lp["ln2_b"], eps), lp, act)
        a = x[:, -1] if post else layer_norm(x[:, -1], params["lnf_g"], params["lnf_b"], eps)
        return head(params, a)

    toks, zs = [], []
    z = run(prompt, 0)
    nxt = argmax_lowest(z)
    toks.append(nxt)
    zs.append(z)
    for s in range(steps):
        feed = nxt if forced is None else np.asarray(forced)[:, s]
        z = run(np.asarray(feed).reshape(B, 1), T0 + s)
        nxt = argmax_lowest(z)
        toks.append(nxt)
        zs.append(z)
    return np.stack(toks, 1), np.stack(zs, 1)
