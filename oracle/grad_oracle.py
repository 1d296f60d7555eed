"""fp64 CPU oracle of the backward pass of the next-token loss through the head,
the final LayerNorm and the embeddings.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may use it.  It shares no code with the HIP library.

The loss is the mean next-token cross-entropy of the forward oracle
(gpt_oracle.forward).  Its gradients are written out from the chain rule, step
by step, in float64:

  [P1] "预训练一个 Mini GPT（1.24 亿参数）", 训练循环: a training step
       back-propagates the cross-entropy to every parameter.
  [P2] "第 25 章 从小 GPT 到 GPT-2：先把模型对上，再谈训练" §25.4: with the
       head tied to the token table E, E's gradient is the sum of the
       contributions of both uses (the output classification and the input
       lookup).
  [P3] "Day 16: 从零组装 MiniGPT——第一次写出完整 GPT 模型": the step runs
       CrossEntropy(logits, Y), then backward, then the optimiser.

Derivatives used (standard calculus, no page prints them):
  * d(mean CE)/dz[n, v] = (softmax(z[n])[v] - [v == y[n]]) / n_valid for rows
    with a target, 0 for rows without one;
  * logits z = a W^T  =>  da = dz W,  dW = dz^T a;
  * LayerNorm y = g * xh + b, xh = (x - mu) / sqrt(var + eps) with the biased
    variance: dx = (gd - mean(gd) - xh * mean(gd * xh)) / sqrt(var + eps) with
    gd = dy * g, dg = sum over rows of dy * xh, db = sum over rows of dy;
  * x0[b, t] = E[idx[b, t]] + P[t]  =>  dE[v] += sum of dx0 over the positions
    holding token v, dP[t] = sum over the batch of dx0[:, t].

  * a block (pre-LN GPT-2): the same rules through both residual paths,
    the two LayerNorms, the GELU (tanh form: derivative of 0.5 z (1 + tanh u)),
    the projections and each causal head: dU = P^T dY, dP = dY U^T,
    dS = P * (dP - rowsum(dP * P)), dQ = dS K / sqrt(D), dK = dS^T Q / sqrt(D).

Pinned by tests/test_oracle_grad.py against central finite differences of the
forward oracle's loss, torch float64 autograd, invariants and planted mistakes.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from oracle import gpt_oracle as O


def ce_head_backward(params: dict, a: np.ndarray, y: np.ndarray):
    """Backward of the mean cross-entropy through the head ([P2] §25.4 tied
    head, or the untied W_head).  a [N, C] final hidden rows, y [N] targets
    (-1 = none).  Returns (dz [N, V], da [N, C], dW_head [V, C], mean loss)."""
    W = params.get("head_w", params["wte"])
    y = np.asarray(y, dtype=np.int64)
    z = a @ W.T
    valid = y >= 0
    n_valid = int(valid.sum())
    if n_valid == 0:
        raise ValueError("no position has a target")
    dz = O.softmax_rows(z)
    rows = np.nonzero(valid)[0]
    dz[rows, y[rows]] -= 1.0
    dz[~valid] = 0.0
    dz /= n_valid
    da = dz @ W
    dW = dz.T @ a
    loss = float(O.cross_entropy_rows(z, y)[valid].sum() / n_valid)
    return dz, da, dW, loss


def layer_norm_backward(x: np.ndarray, g: np.ndarray, dy: np.ndarray, eps: float = 1e-5):
    """Gradient of y = g * (x - mean) / sqrt(var + eps) + b (biased variance,
    over the last axis) for an upstream gradient dy.  Returns (dx, dg, db)."""
    C = x.shape[-1]
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + eps)
    xh = (x - mu) * r
    gd = dy * g
    dx = r * (gd - gd.mean(axis=-1, keepdims=True) - xh * (gd * xh).mean(axis=-1, keepdims=True))
    dg = (dy * xh).reshape(-1, C).sum(axis=0)
    db = dy.reshape(-1, C).sum(axis=0)
    return dx, dg, db


def head_backward(params: dict, x: np.ndarray, y: np.ndarray, eps: float = 1e-5) -> dict:
    """Backward from the rows the final LayerNorm reads (pre-LN models) or the
    final hidden rows themselves (post-LN models, which have no final
    LayerNorm) to the loss.  x [N, C], y [N].  Returns a dict with dx [N, C],
    the head matrix's gradient under "head" (the token table's share when the
    head is tied), "lnf_g" / "lnf_b" (pre-LN only) and "loss"."""
    post = params.get("norm", "pre") == "post"
    a = x if post else O.layer_norm(x, params["lnf_g"], params["lnf_b"], eps)
    _, da, dW, loss = ce_head_backward(params, a, y)
    out = {"head": dW, "loss": loss}
    if post:
        out["dx"] = da
    else:
        out["dx"], out["lnf_g"], out["lnf_b"] = layer_norm_backward(x, params["lnf_g"], da, eps)
    return out


def embedding_backward(idx: np.ndarray, dx0: np.ndarray, vocab: int, ctx: int):
    """Gradients of x0[b, t] = E[idx[b, t]] + P[t] for an upstream dx0 [B, T, C]:
    (dE [vocab, C] summing the rows of every position holding a token,
    dP [ctx, C] summing over the batch; positions >= T get 0)."""
    idx = np.asarray(idx)
    B, T = idx.shape
    C = dx0.shape[-1]
    dE = np.zeros((vocab, C))
    for b in range(B):
        for t in range(T):
            dE[idx[b, t]] += dx0[b, t]
    dP = np.zeros((ctx, C))
    dP[:T] = dx0.sum(axis=0)
    return dE, dP


def grads_no_blocks(params: dict, idx: np.ndarray, targets: Optional[np.ndarray] = None,
                    eps: float = 1e-5) -> dict:
    """Every parameter gradient of the mean next-token loss of a model with no
    blocks: embedding -> (final LayerNorm) -> head.  With a tied head the
    token table's gradient is the head share plus the lookup share ([P2]
    §25.4).  Returns {"wte", "wpe", "lnf_g", "lnf_b" (pre-LN), "head_w"
    (untied), "loss"}."""
    if params["layers"]:
        raise ValueError("model has blocks")
    idx = np.asarray(idx)
    B, T = idx.shape
    y = O.derived_targets(idx) if targets is None else np.asarray(targets, dtype=np.int64)
    x0 = O.embed(params, idx)
    C = x0.shape[-1]
    hb = head_backward(params, x0.reshape(B * T, C), y.reshape(B * T), eps)
    dE, dP = embedding_backward(idx, hb["dx"].reshape(B, T, C), params["wte"].shape[0], params["wpe"].shape[0])
    g = {"wpe": dP, "loss": hb["loss"]}
    if "head_w" in params:
        g["wte"] = dE
        g["head_w"] = hb["head"]
    else:
        g["wte"] = dE + hb["head"]
    if "lnf_g" in hb:
        g["lnf_g"], g["lnf_b"] = hb["lnf_g"], hb["lnf_b"]
    return g


# ----------------------------------------------------------------------------
# Block backward (pre-LN GPT-2 blocks)
# ----------------------------------------------------------------------------
def gelu_tanh_grad(z: np.ndarray) -> np.ndarray:
    """d/dz of 0.5 z (1 + tanh u), u = sqrt(2/pi) (z + 0.044715 z^3)."""
    c = math.sqrt(2.0 / math.pi)
    t = np.tanh(c * (z + 0.044715 * z ** 3))
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c * (1.0 + 3 * 0.044715 * z * z)


def gelu_erf_grad(z: np.ndarray) -> np.ndarray:
    """d/dz of z Phi(z) = Phi(z) + z phi(z)."""
    from scipy.special import erf
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def attention_backward(q: np.ndarray, k: np.ndarray, u: np.ndarray, dy: np.ndarray):
    """One causal head y = softmax(q k^T / sqrt(D) + M) u: returns (dq, dk, du).
    With P the softmax: du = P^T dy; dP = dy u^T; dS = P * (dP - rowsum(dP * P));
    dq = dS k / sqrt(D); dk = dS^T q / sqrt(D)."""
    T, D = q.shape
    s = (q @ k.T) / math.sqrt(D)
    s = np.where(np.triu(np.ones((T, T), dtype=bool), k=1), -np.inf, s)
    p = O.softmax_rows(s)
    du = p.T @ dy
    dp = dy @ u.T
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
    return ds @ k / math.sqrt(D), ds.T @ q / math.sqrt(D), du


def block_backward(x: np.ndarray, lp: dict, dy: np.ndarray, n_head: int, eps: float = 1e-5,
                   act: str = "tanh"):
    """Gradient of a pre-norm block out = x1 + mlp(LN2(x1)), x1 = x + attn(LN1(x))
    for the upstream dy = d loss / d out.  x, dy [B, T, C].  Recomputes the
    block's forward, then applies the chain rule in reverse.  Returns (dx,
    grads keyed like lp)."""
    B, T, C = x.shape
    D = C // n_head
    g = {}
    a1 = O.layer_norm(x, lp["ln1_g"], lp["ln1_b"], eps)
    qkv = O.linear(a1, lp["attn_w"], lp["attn_b"])
    heads = lambda z: z.reshape(B, T, n_head, D).transpose(0, 2, 1, 3)
    qh, kh, uh = heads(qkv[..., :C]), heads(qkv[..., C:2 * C]), heads(qkv[..., 2 * C:])
    yh = np.empty_like(qh)
    for b in range(B):
        for h in range(n_head):
            yh[b, h] = O.causal_attention(qh[b, h], kh[b, h], uh[b, h])
    o = yh.transpose(0, 2, 1, 3).reshape(B, T, C)
    x1 = x + O.linear(o, lp["proj_w"], lp["proj_b"])
    a2 = O.layer_norm(x1, lp["ln2_g"], lp["ln2_b"], eps)
    z = O.linear(a2, lp["fc_w"], lp["fc_b"])
    hmid = O.activation(z, act)
    flat = lambda t: t.reshape(-1, t.shape[-1])
    # MLP
    g["fcproj_w"] = flat(dy).T @ flat(hmid)
    g["fcproj_b"] = flat(dy).sum(axis=0)
    dz = (dy @ lp["fcproj_w"]) * (gelu_erf_grad(z) if act == "erf" else gelu_tanh_grad(z))
    g["fc_w"] = flat(dz).T @ flat(a2)
    g["fc_b"] = flat(dz).sum(axis=0)
    dx1_ln, g["ln2_g"], g["ln2_b"] = layer_norm_backward(x1, lp["ln2_g"], dz @ lp["fc_w"], eps)
    dx1 = dy + dx1_ln
    # attention
    g["proj_w"] = flat(dx1).T @ flat(o)
    g["proj_b"] = flat(dx1).sum(axis=0)
    doh = heads(dx1 @ lp["proj_w"])
    dq, dk, du = np.empty_like(qh), np.empty_like(kh), np.empty_like(uh)
    for b in range(B):
        for h in range(n_head):
            dq[b, h], dk[b, h], du[b, h] = attention_backward(qh[b, h], kh[b, h], uh[b, h], doh[b, h])
    merge = lambda t: t.transpose(0, 2, 1, 3).reshape(B, T, C)
    dqkv = np.concatenate([merge(dq), merge(dk), merge(du)], axis=-1)
    g["attn_w"] = flat(dqkv).T @ flat(a1)
    g["attn_b"] = flat(dqkv).sum(axis=0)
    dx_ln, g["ln1_g"], g["ln1_b"] = layer_norm_backward(x, lp["ln1_g"], dqkv @ lp["attn_w"], eps)
    return dx1 + dx_ln, g


def grads_full(params: dict, idx: np.ndarray, n_head: int, targets: Optional[np.ndarray] = None,
               eps: float = 1e-5) -> dict:
    """Every parameter gradient of the mean next-token loss of a pre-LN GPT-2
    model: forward keeping each block's input, head backward, the blocks in
    reverse, then the embeddings (the tied table's two shares summed, [P2]
    §25.4).  Returns {"wte", "wpe", "layers": [grads per block], "lnf_g",
    "lnf_b", "head_w" (untied), "loss"}."""
    if params.get("norm", "pre") != "pre":
        raise ValueError("pre-LN blocks only")
    idx = np.asarray(idx)
    B, T = idx.shape
    act = params.get("act", "tanh")
    y = O.derived_targets(idx) if targets is None else np.asarray(targets, dtype=np.int64)
    xs = [O.embed(params, idx)]
    for lp in params["layers"]:
        xs.append(O.block(xs[-1], lp, n_head, eps, act=act))
    C = xs[0].shape[-1]
    hb = head_backward(params, xs[-1].reshape(B * T, C), y.reshape(B * T), eps)
    dx = hb["dx"].reshape(B, T, C)
    layers = [None] * len(params["layers"])
    for l in range(len(params["layers"]) - 1, -1, -1):
        dx, layers[l] = block_backward(xs[l], params["layers"][l], dx, n_head, eps, act)
    dE, dP = embedding_backward(idx, dx, params["wte"].shape[0], params["wpe"].shape[0])
    g = {"wpe": dP, "layers": layers, "lnf_g": hb["lnf_g"], "lnf_b": hb["lnf_b"], "loss": hb["loss"]}
    if "head_w" in params:
        g["wte"], g["head_w"] = dE, hb["head"]
    else:
        g["wte"] = dE + hb["head"]
    return g
