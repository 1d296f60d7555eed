"""fp64 CPU oracle of the LLaMA-style decoder-only model: RMSNorm, RoPE on
queries and keys, grouped-query attention, SwiGLU feed-forward, no position
table and no biases.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may use it.  It shares no code with the HIP library.

Sources (web pages, cited by title and section):
  [P4] "02 GPT 架构——Decoder-Only 的自回归语言模型": §5.2 RoPE (the 2-D
       rotation of each adjacent pair (2i, 2i+1) by the angle m * theta_i,
       theta_i = 10000^(-2i/d); the rotated dot product depends only on m - n),
       §6.1 the LLaMA block (pre-norm RMSNorm, attention with RoPE, residual,
       RMSNorm, SwiGLU SiLU(x W1) * (x W3) then the down projection, residual),
       §6.2 GQA (groups of query heads share one K/V head; MQA: one K/V head),
       §6.3 assembly (token embedding, L blocks, final RMSNorm, head);
  [P5] "GPT-1学习笔记：“预训练+微调”范式" §10.2: RMSNorm drops the mean
       centring and the bias of LayerNorm; SwiGLU(x) = (W_a x) * Swish(W_b x)
       with Swish(x) = x sigma(x).

Readings where the pages leave a step open (each listed with its pin in the
project's design notes): d in theta_i is the head width D; RMSNorm is
g * x / sqrt(mean(x^2) + eps) with the same eps as the LayerNorm models;
the projections carry no bias; attention scales by 1/sqrt(D) and masks the
future as the GPT-2 model does; query head h reads K/V head h // (H / Hkv);
ALiBi (the page's alternative, [P4] §5.3) replaces the rotation with the
distance bias -m_h |i - j|, slopes m_h = 2^(-8 (h+1) / H).
Weight storage (a layout choice, not arithmetic): wqkv_w stacks the rows of
W_q [H*D, C], W_k [Hkv*D, C], W_v [Hkv*D, C]; w13_w interleaves the rows of
W1 (gate, even rows) and W3 (up, odd rows).
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from oracle import gpt_oracle as O


def param_count(vocab: int, n_embd: int, n_layer: int, n_head: int, n_kv_head: int, n_ff: int,
                untied: bool = False) -> int:
    """Per block: two RMSNorm gains 2C, W_q and W_o 2C^2, W_k and W_v
    2 C Hkv D, the three SwiGLU matrices 3 C F; plus the token table V C, the
    final RMSNorm C and, untied, the head V C."""
    C, F = n_embd, n_ff
    D = C // n_head
    per = 2 * C + 2 * C * C + 2 * C * n_kv_head * D + 3 * C * F
    return n_layer * per + vocab * C + C + (vocab * C if untied else 0)


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """g * x / sqrt(mean(x^2) + eps) over the last axis ([P5] §10.2: no mean
    centring, no bias)."""
    return g * x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)


def rope(x: np.ndarray, pos: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """Rotate each adjacent pair (x[2i], x[2i+1]) of the last axis by the angle
    pos * theta^(-2i/D) ([P4] §5.2): x'[2i] = cos x[2i] - sin x[2i+1],
    x'[2i+1] = sin x[2i] + cos x[2i+1].  x [..., T, D], pos [T]."""
    D = x.shape[-1]
    i = np.arange(D // 2)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta ** (-2.0 * i / D)   # [T, D/2]
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = c * xe - s * xo
    out[..., 1::2] = s * xe + c * xo
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU = Swish: z * sigma(z) ([P5] §10.2)."""
    return z / (1.0 + np.exp(-z))


def swiglu_mlp(a: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """W2 (SiLU(a W1^T) * (a W3^T)) ([P4] §6.1), W1 = even rows of w13, W3 = odd rows."""
    gate = a @ w13[0::2].T
    up = a @ w13[1::2].T
    return (silu(gate) * up) @ w2.T


def alibi_slopes(H: int) -> np.ndarray:
    """Per-head ALiBi slopes, a geometric series ([P4] §5.3 gives no
    formula; the reading taken is the ALiBi paper's m_h = 2^(-8 (h+1) / H))."""
    return 2.0 ** (-8.0 * (np.arange(H) + 1) / H)


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, slopes: Optional[np.ndarray] = None) -> np.ndarray:
    """Causal attention where query head h reads K/V head h // (H / Hkv)
    ([P4] §6.2).  q [B, H, T, D], k, v [B, Hkv, Tk, D] with the queries at the
    last T of the Tk key positions.  With ALiBi slopes the scores are
    q.k / sqrt(D) - m_h |i - j| ([P4] §5.3).  Returns [B, H, T, D]."""
    B, H, T, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    grp = H // Hkv
    y = np.empty_like(q)
    off = Tk - T
    dist = (off + np.arange(T))[:, None] - np.arange(Tk)[None, :]     # i - j
    for b in range(B):
        for h in range(H):
            s = q[b, h] @ k[b, h // grp].T / math.sqrt(D)            # [T, Tk]
            if slopes is not None:
                s = s - slopes[h] * np.abs(dist)
            mask = np.arange(Tk)[None, :] > (off + np.arange(T))[:, None]
            s = np.where(mask, -np.inf, s)
            y[b, h] = O.softmax_rows(s) @ v[b, h // grp]
    return y


def _split_qkv(x_a: np.ndarray, lp: dict, H: int, Hkv: int, D: int):
    B, T, C = x_a.shape
    qkv = x_a @ lp["wqkv_w"].T
    q = qkv[..., :H * D].reshape(B, T, H, D).transpose(0, 2, 1, 3)
    k = qkv[..., H * D:(H + Hkv) * D].reshape(B, T, Hkv, D).transpose(0, 2, 1, 3)
    v = qkv[..., (H + Hkv) * D:].reshape(B, T, Hkv, D).transpose(0, 2, 1, 3)
    return q, k, v


def block(x: np.ndarray, lp: dict, H: int, Hkv: int, theta: float, eps: float,
          cache: Optional[dict] = None, pos0: int = 0, alibi: bool = False) -> np.ndarray:
    """One LLaMA block ([P4] §6.1) on x [B, T, C] at positions pos0 .. pos0+T-1.
    With a cache dict (keys 'k', 'v' of [B, Hkv, t, D]) the rotated keys and
    the values are appended and attention reads every cached position.  alibi:
    no rotation; the scores carry the ALiBi distance bias instead ([P4] §5.3)."""
    B, T, C = x.shape
    D = C // H
    a = rms_norm(x, lp["rms1_g"], eps)
    q, k, v = _split_qkv(a, lp, H, Hkv, D)
    pos = pos0 + np.arange(T)
    if not alibi:
        q, k = rope(q, pos, theta), rope(k, pos, theta)
    if cache is not None:
        if "k" in cache:
            k = np.concatenate([cache["k"], k], axis=2)
            v = np.concatenate([cache["v"], v], axis=2)
        cache["k"], cache["v"] = k, v
    y = gqa_attention(q, k, v, alibi_slopes(H) if alibi else None).transpose(0, 2, 1, 3).reshape(B, T, C)
    x = x + y @ lp["wo_w"].T
    return x + swiglu_mlp(rms_norm(x, lp["rms2_g"], eps), lp["w13_w"], lp["w2_w"])


def final_hidden(params: dict, idx: np.ndarray, H: int, eps: float = 1e-5) -> np.ndarray:
    """Token embedding (no position table), the blocks, final RMSNorm ([P4] §6.3)."""
    x = params["wte"][np.asarray(idx)]
    for lp in params["layers"]:
        x = block(x, lp, H, params["n_kv_head"], params["rope_theta"], eps, alibi=params.get("alibi", False))
    return rms_norm(x, params["rmsf_g"], eps)


def forward(params: dict, idx: np.ndarray, H: int, eps: float = 1e-5, targets: Optional[np.ndarray] = None,
            want_logits: bool = True) -> Tuple[Optional[np.ndarray], np.ndarray, float]:
    """Logits (head tied to wte unless the params carry head_w), per-token
    next-token cross-entropy and its mean over positions with a target; the
    same loss and target rules as the GPT-2 oracle."""
    idx = np.asarray(idx)
    B, T = idx.shape
    a = final_hidden(params, idx, H, eps)
    y = O.derived_targets(idx) if targets is None else np.asarray(targets, dtype=np.int64)
    z = O.head(params, a.reshape(B * T, -1))
    tok = O.cross_entropy_rows(z, y.reshape(-1))
    valid = y.reshape(-1) >= 0
    mean = float(tok[valid].sum() / valid.sum()) if valid.any() else float("nan")
    return (z.reshape(B, T, -1) if want_logits else None), tok.reshape(B, T), mean


def greedy_recompute(params: dict, prompt: np.ndarray, steps: int, H: int, eps: float = 1e-5):
    """Greedy decoding by re-running the whole sequence each step."""
    seq = np.asarray(prompt)
    toks, lasts = [], []
    for _ in range(steps + 1):
        a = final_hidden(params, seq, H, eps)[:, -1]
        z = O.head(params, a)
        t = O.argmax_lowest(z)
        toks.append(t)
        lasts.append(z)
        seq = np.concatenate([seq, t[:, None]], axis=1)
    return np.stack(toks, 1), np.stack(lasts, 1)


def greedy_cached(params: dict, prompt: np.ndarray, steps: int, H: int, eps: float = 1e-5,
                  forced: Optional[np.ndarray] = None):
    """Greedy decoding with per-layer K/V caches (rotated keys, Hkv heads).
    forced [B, steps]: feed these tokens instead of the argmax (teacher
    forcing, to compare logits along another decoder's history)."""
    prompt = np.asarray(prompt)
    caches = [dict() for _ in params["layers"]]
    pos0, toks, lasts = 0, [], []
    cur = prompt
    for it in range(steps + 1):
        x = params["wte"][cur]
        for lp, c in zip(params["layers"], caches):
            x = block(x, lp, H, params["n_kv_head"], params["rope_theta"], eps, cache=c, pos0=pos0,
                      alibi=params.get("alibi", False))
        pos0 += cur.shape[1]
        z = O.head(params, rms_norm(x[:, -1], params["rmsf_g"], eps))
        t = O.argmax_lowest(z)
        toks.append(t)
        lasts.append(z)
        cur = (t if forced is None or it >= steps else np.asarray(forced)[:, it])[:, None]
    return np.stack(toks, 1), np.stack(lasts, 1)
