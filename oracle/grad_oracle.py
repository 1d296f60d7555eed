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

Pinned by tests/test_oracle_grad.py against central finite differences of the
forward oracle's loss, torch float64 autograd, invariants and planted mistakes.
"""
from __future__ import annotations

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
