"""Next-token sampling from one row of logits: repetition penalty, temperature,
top-k and top-p (nucleus), then one draw.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may use it.  It shares no code with the HIP library.

Sources (web pages, cited by title and section):
  [P1] "预训练一个 Mini GPT（1.24 亿参数）", 构建它 第7步 (文本生成): logits of
       the last position divided by the temperature, softmax with the maximum
       subtracted, one draw with np.random.choice (inverse CDF in float64);
       temperature 0 is the greedy choice.
  [P2] "第 25 章 从小 GPT 到 GPT-2", §25.7: top-k = 50 as the course setting,
       draws from the relative probabilities of the kept candidates.
  [P4] "02 GPT 架构——Decoder-Only 的自回归语言模型", 第 8 章 §8.1 temperature,
       §8.2 top-k, §8.3 top-p (sort by probability, accumulate until the sum
       reaches p), §8.4 repetition penalty (a logit of a token that already
       appeared is divided by alpha when positive, multiplied when negative),
       and the remark that the strategies are used together.
  [P5] "GPT-1学习笔记", §6.2: temperature, top-k (renormalise the k largest),
       top-p (the smallest set whose cumulative probability reaches p).

Readings (the pages leave these open):
  * order of the steps: penalty, temperature, top-k, top-p, draw;
  * precision: float64 throughout, the precision of [P1]'s numpy sampler
    (the logits themselves are the values the model produced, bf16 or fp32,
    upcast exactly): the penalised logit, the key z'/T, each candidate's
    unnormalised probability weight exp(key - max key), the masses, the
    thresholds and the draw;
  * the nucleus is taken of the distribution left by top-k (renormalised),
    as the smallest prefix in descending probability whose mass is >= p * Z;
  * candidates are ordered by descending weight, equal weights by ascending
    index; this order decides which of several equally probable tokens top-k
    and top-p keep, and it is the order the inverse CDF walks: the draw u in
    [0, 1) returns the first candidate whose cumulative mass exceeds
    u * (mass of the nucleus);
  * temperature <= 0 is the greedy choice (lowest index among equal maxima);
  * the uniform u is an input (the caller's random stream), one per row.

Every function is pinned by CPU tests (tests/test_oracle_sampling.py) against
closed forms (softmax frequencies of a stratified set of draws), brute force
over small vocabularies and the worked penalty rule of [P4] §8.4.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def penalize(z: np.ndarray, seen: Optional[np.ndarray], alpha: float) -> np.ndarray:
    """[P4] §8.4: z/alpha where the token appeared and z > 0, z*alpha where it
    appeared and z < 0, unchanged otherwise (float64)."""
    z = np.asarray(z, dtype=np.float64)
    if seen is None or alpha == 1.0:
        return z.copy()
    a = np.float64(alpha)
    seen = np.asarray(seen, dtype=bool)
    out = z.copy()
    pos = seen & (z > 0)
    neg = seen & (z < 0)
    out[pos] = z[pos] / a
    out[neg] = z[neg] * a
    return out


def candidate_order(w: np.ndarray) -> np.ndarray:
    """Indices by descending weight, ascending index among equal weights."""
    V = w.size
    return np.lexsort((np.arange(V), -np.asarray(w, dtype=np.float64)))


def keys(z: np.ndarray, seen: Optional[np.ndarray], temperature: float, alpha: float = 1.0) -> np.ndarray:
    """key = z'/T ([P1] 第7步, [P4] §8.1), z' the penalised logits (float64)."""
    return penalize(z, seen, alpha) / np.float64(temperature)


def weights(z: np.ndarray, seen: Optional[np.ndarray], temperature: float, alpha: float = 1.0) -> np.ndarray:
    """Unnormalised probability weights exp(key - max key) (float64): the
    softmax numerator with the maximum subtracted ([P1] 第7步)."""
    key = keys(z, seen, temperature, alpha)
    return np.exp(key - key.max())


def filtered(z: np.ndarray, seen: Optional[np.ndarray], temperature: float, top_k: int, top_p: float,
             alpha: float = 1.0):
    """The candidates left after penalty, temperature, top-k and top-p, in
    candidate order, with their float64 weights."""
    w64 = weights(z, seen, temperature, alpha)
    order = candidate_order(w64)
    V = w64.size
    cand = order[:top_k] if 0 < top_k < V else order                # [P4] §8.2, [P5] §6.2
    w = w64[cand]
    if top_p < 1.0:                                                 # [P4] §8.3, [P5] §6.2
        cum = np.cumsum(w)
        n = int(np.searchsorted(cum, top_p * cum[-1], side="left")) + 1   # first prefix with mass >= p Z
        cand, w = cand[:n], w[:n]
    return cand, w


def sample_row(z: np.ndarray, seen: Optional[np.ndarray], temperature: float, top_k: int, top_p: float,
               alpha: float, u: float) -> int:
    """One next token for one row of logits, from the uniform draw u in [0, 1)."""
    if temperature <= 0:
        return int(np.argmax(penalize(z, seen, alpha)))             # first maximum: lowest index
    cand, w = filtered(z, seen, temperature, top_k, top_p, alpha)
    r = float(u) * float(w.sum())
    pos = int(np.searchsorted(np.cumsum(w), r, side="right"))       # first cumulative mass > r
    return int(cand[min(pos, len(cand) - 1)])


def sample_rows(z: np.ndarray, seen: Optional[np.ndarray], temperature: float, top_k: int, top_p: float,
                alpha: float, u: np.ndarray) -> np.ndarray:
    """sample_row over the rows of z [B, V] (seen [B, V] bool or None, u [B])."""
    return np.array([sample_row(z[b], None if seen is None else seen[b], temperature, top_k, top_p, alpha,
                                float(u[b])) for b in range(z.shape[0])], dtype=np.int64)
