"""Seeded synthetic inputs: model configurations, parameter tensors and token ids.

This module is the only code shared by the fp64 oracle side and the HIP side.
It holds no arithmetic of the forward pass: it draws random numbers, rounds
them to the storage dtype and packs them in the fixed parameter order that the
C library's `gpt_param_offsets` also implements (the two are checked against
each other by a CPU test).

Initialisation follows the pages: weights N(0, 0.02) ("预训练一个 Mini GPT",
第1步 嵌入层; "第 25 章 从小 GPT 到 GPT-2", §25.6), biases zero, LayerNorm gain
one and bias zero.  A second "stress" init makes every bias and LayerNorm
parameter non-trivial so that parity tests exercise each term.

Packing order of the flat parameter blob (one shared token table, no separate
head tensor, because the head is tied to it, §25.4 of the GPT-2 chapter):

    wte[V,C], wpe[ctx,C],
    per layer: ln1_g[C], ln1_b[C], attn_w[3C,C], attn_b[3C], proj_w[C,C],
               proj_b[C], ln2_g[C], ln2_b[C], fc_w[F,C], fc_b[F],
               fcproj_w[C,F], fcproj_b[C],
    lnf_g[C], lnf_b[C]

Every matrix is stored row-major as [out, in], so a linear layer is
y = x W^T + b.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

F32 = 0
BF16 = 1


@dataclasses.dataclass(frozen=True)
class GPTConfig:
    vocab: int
    ctx: int
    n_embd: int
    n_head: int
    n_layer: int
    n_ff: int
    ln_eps: float = 1e-5
    dtype: int = F32  # 0 = fp32, 1 = bf16 (storage and MFMA operand type)
    act: int = 0      # 0 = tanh GELU (GPT-2), 1 = exact erf GELU
    post_ln: int = 0  # 0 = pre-LN blocks + ln_f (GPT-2), 1 = post-LN blocks, no ln_f (GPT-1)
    untied: int = 0   # 0 = head tied to the token table, 1 = separate head matrix [V, C]
    arch: int = 0     # 0 = GPT-2 blocks, 1 = LLaMA-style blocks (RMSNorm, RoPE, SwiGLU, GQA, no biases)
    n_kv_head: int = 0  # LLaMA: K/V heads shared by groups of query heads (0 = n_head)
    rope_theta: float = 10000.0
    alibi: int = 0      # LLaMA-style only: ALiBi distance bias in place of RoPE

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head

    @property
    def kv_heads(self) -> int:
        return self.n_kv_head or self.n_head


# Named workloads.  Ids: 1 micro fp32, 2 MiniGPT fp32, 3 GPT-2 124M bf16
# (B=8,T=1024), 4 GPT-2 124M bf16 at B=32 without logits, 5 GPT-2 decode.
MICRO = GPTConfig(vocab=17, ctx=12, n_embd=16, n_head=2, n_layer=2, n_ff=64, dtype=F32)
MINI = GPTConfig(vocab=5000, ctx=128, n_embd=128, n_head=4, n_layer=4, n_ff=512, dtype=F32)
GPT2 = GPTConfig(vocab=50257, ctx=1024, n_embd=768, n_head=12, n_layer=12, n_ff=3072, dtype=BF16)
GPT2_F32 = dataclasses.replace(GPT2, dtype=F32)
# LLaMA-style blocks at the GPT-2 width: 12 query heads sharing 4 K/V heads,
# SwiGLU width 8/3 C = 2048, tied head over the GPT-2 vocabulary
LLAMA_124 = GPTConfig(vocab=50257, ctx=1024, n_embd=768, n_head=12, n_layer=12, n_ff=2048, dtype=BF16, arch=1,
                      n_kv_head=4)

WORKLOADS = {
    1: dict(cfg=MICRO, B=4, T=12, name="micro-fp32 V17 C16 H2 L2 B4 T12"),
    2: dict(cfg=MINI, B=4, T=64, name="minigpt-fp32 V5000 C128 H4 L4 B4 T64"),
    3: dict(cfg=GPT2, B=8, T=1024, name="gpt2-124M-bf16 B8 T1024 fwd+loss"),
    4: dict(cfg=GPT2, B=32, T=1024, name="gpt2-124M-bf16 B32 T1024 fused CE, no logits"),
    5: dict(cfg=GPT2, B=64, T=128, name="gpt2-124M-bf16 decode B64 prompt128 +128 greedy"),
    6: dict(cfg=LLAMA_124, B=8, T=1024, name="llama-style-bf16 C768 H12 KV4 L12 F2048 B8 T1024 fwd+loss"),
}

LAYER_FIELDS = ("ln1_g", "ln1_b", "attn_w", "attn_b", "proj_w", "proj_b",
                "ln2_g", "ln2_b", "fc_w", "fc_b", "fcproj_w", "fcproj_b")


LLAMA_FIELDS = ("rms1_g", "wqkv_w", "wo_w", "rms2_g", "w13_w", "w2_w")


def layer_shapes(cfg: GPTConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    C, F = cfg.n_embd, cfg.n_ff
    if cfg.arch == 1:
        # wqkv: rows of W_q (H*D), then W_k and W_v (Hkv*D each); w13: rows
        # interleaved, 2j = gate (W1) row j, 2j+1 = up (W3) row j
        D = cfg.head_dim
        return [("rms1_g", (C,)), ("wqkv_w", ((cfg.n_head + 2 * cfg.kv_heads) * D, C)), ("wo_w", (C, C)),
                ("rms2_g", (C,)), ("w13_w", (2 * F, C)), ("w2_w", (C, F))]
    return [("ln1_g", (C,)), ("ln1_b", (C,)), ("attn_w", (3 * C, C)), ("attn_b", (3 * C,)),
            ("proj_w", (C, C)), ("proj_b", (C,)), ("ln2_g", (C,)), ("ln2_b", (C,)),
            ("fc_w", (F, C)), ("fc_b", (F,)), ("fcproj_w", (C, F)), ("fcproj_b", (C,))]


def blob_layout(cfg: GPTConfig) -> List[Tuple[str, Tuple[int, ...], int]]:
    """(name, shape, element offset) for every tensor of the blob, in packing order."""
    out = []
    off = 0

    def add(name, shape):
        nonlocal off
        out.append((name, shape, off))
        off += int(np.prod(shape))

    add("wte", (cfg.vocab, cfg.n_embd))
    if cfg.arch == 0:
        add("wpe", (cfg.ctx, cfg.n_embd))
    for l in range(cfg.n_layer):
        for name, shape in layer_shapes(cfg):
            add(f"h{l}.{name}", shape)
    if cfg.arch == 1:
        add("rmsf_g", (cfg.n_embd,))
    elif not cfg.post_ln:
        add("lnf_g", (cfg.n_embd,))
        add("lnf_b", (cfg.n_embd,))
    if cfg.untied:
        add("head_w", (cfg.vocab, cfg.n_embd))
    out.append(("__end__", (), off))
    return out


def blob_numel(cfg: GPTConfig) -> int:
    return blob_layout(cfg)[-1][2]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with round-to-nearest-even, returned as fp32 holding the bf16 value."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) & 0xFFFF
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_params(cfg: GPTConfig, seed: int = 42, cfg_id: int = 0, init: str = "bench",
                zero_residual_proj: bool = False) -> Dict[str, np.ndarray]:
    """Draw every parameter as fp32 and round it to cfg.dtype.

    Returned arrays are float32 holding values exactly representable in the
    storage dtype, keyed as in the blob ("wte", "wpe", "h{l}.attn_w", ..., "lnf_b").
    init="bench": W ~ N(0,0.02), biases 0, gains 1, LN biases 0.
    init="stress": additionally biases ~ N(0,0.02), gains ~ 1+N(0,0.1), LN biases ~ N(0,0.02).
    """
    rng = np.random.default_rng((seed, cfg_id, 0))
    p: Dict[str, np.ndarray] = {}
    std = 0.02
    stress = init == "stress"
    for name, shape, _ in blob_layout(cfg)[:-1]:
        base = name.split(".")[-1]
        if base in ("wte", "wpe") or base.endswith("_w"):
            v = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
        elif base.endswith("_g"):
            v = np.ones(shape, np.float32)
            if stress:
                v = v + rng.standard_normal(shape, dtype=np.float32) * np.float32(0.1)
        else:  # biases and LayerNorm offsets
            v = np.zeros(shape, np.float32)
            if stress:
                v = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
        if zero_residual_proj and base in ("proj_w", "proj_b", "fcproj_w", "fcproj_b"):
            v = np.zeros(shape, np.float32)
        p[name] = v.astype(np.float32)
    if cfg.dtype == BF16:
        p = {k: round_bf16(v) for k, v in p.items()}
    return p


def pack(cfg: GPTConfig, params: Dict[str, np.ndarray]) -> np.ndarray:
    """Flat blob in packing order: float32 for fp32 configs, uint16 bf16 bits for bf16."""
    flat = np.empty(blob_numel(cfg), np.float32)
    for name, shape, off in blob_layout(cfg)[:-1]:
        a = params[name]
        assert a.shape == shape, (name, a.shape, shape)
        flat[off:off + a.size] = a.reshape(-1)
    if cfg.dtype == BF16:
        return f32_to_bf16_bits(flat)
    return flat


def unpack_f64(cfg: GPTConfig, params: Dict[str, np.ndarray]) -> dict:
    """Nested float64 view for the oracle: {'wte','wpe','layers':[{...}], 'lnf_g','lnf_b'}
    (no ln_f for post-LN configurations, 'head_w' for an untied head), plus the
    variant names 'act' ('tanh' or 'erf') and 'norm' ('pre' or 'post')."""
    if cfg.arch == 1:
        out = {"arch": "llama", "wte": params["wte"].astype(np.float64), "rmsf_g": params["rmsf_g"].astype(np.float64),
               "n_kv_head": cfg.kv_heads, "rope_theta": float(cfg.rope_theta), "alibi": bool(cfg.alibi),
               "layers": []}
        if cfg.untied:
            out["head_w"] = params["head_w"].astype(np.float64)
        for l in range(cfg.n_layer):
            out["layers"].append({f: params[f"h{l}.{f}"].astype(np.float64) for f in LLAMA_FIELDS})
        return out
    out = {"wte": params["wte"].astype(np.float64), "wpe": params["wpe"].astype(np.float64),
           "layers": [], "act": "erf" if cfg.act else "tanh", "norm": "post" if cfg.post_ln else "pre"}
    if not cfg.post_ln:
        out["lnf_g"] = params["lnf_g"].astype(np.float64)
        out["lnf_b"] = params["lnf_b"].astype(np.float64)
    if cfg.untied:
        out["head_w"] = params["head_w"].astype(np.float64)
    for l in range(cfg.n_layer):
        out["layers"].append({f: params[f"h{l}.{f}"].astype(np.float64) for f in LAYER_FIELDS})
    return out


def make_ids(cfg: GPTConfig, B: int, T: int, seed: int = 42, cfg_id: int = 0) -> np.ndarray:
    """Token ids uniform in [0, V), int32 [B, T]."""
    rng = np.random.default_rng((seed, cfg_id, 1))
    return rng.integers(0, cfg.vocab, size=(B, T), dtype=np.int32)
