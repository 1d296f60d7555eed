"""ctypes binding of libgptmi.so (the C ABI in include/gptmi.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI.  torch supplies device memory and the stream
(`torch.cuda.current_stream().cuda_stream`).  There is no fallback: if the
library is missing, `load()` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, unless GPTMI_LIB names another copy of the library
LIB_PATH = os.environ.get("GPTMI_LIB") or os.path.join(HERE, "libgptmi.so")

GPT_OK = 0
STATUS = {0: "GPT_OK", -1: "GPT_ERR_NULL", -2: "GPT_ERR_CONFIG", -3: "GPT_ERR_SEQ_TOO_LONG",
          -4: "GPT_ERR_SHAPE", -5: "GPT_ERR_WORKSPACE", -6: "GPT_ERR_DTYPE", -7: "GPT_ERR_HIP"}
GPT_ERR_NULL, GPT_ERR_CONFIG, GPT_ERR_SEQ_TOO_LONG, GPT_ERR_SHAPE, GPT_ERR_WORKSPACE = -1, -2, -3, -4, -5

# Every exported function and its ctypes signature.
_c_int, _c_i64, _vp, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t


class gpt_config(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("ctx", ctypes.c_int32), ("n_embd", ctypes.c_int32),
                ("n_head", ctypes.c_int32), ("n_layer", ctypes.c_int32), ("n_ff", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("dtype", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("post_ln", ctypes.c_int32), ("untied_head", ctypes.c_int32), ("arch", ctypes.c_int32),
                ("n_kv_head", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("alibi", ctypes.c_int32)]


class gpt_sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float),
                ("repetition_penalty", ctypes.c_float)]


_CFG = ctypes.POINTER(gpt_config)
SIGNATURES = {
    "gpt_param_count": (_c_i64, [_CFG]),
    "gpt_param_offsets": (_c_int, [_CFG, ctypes.POINTER(ctypes.c_int64), _c_int]),
    "gpt_workspace_bytes": (_c_int, [_CFG, _c_int, _c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "gpt_forward": (_c_int, [_CFG, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gpt_forward_ld": (_c_int, [_CFG, _vp, _vp, _c_int, _c_int, _vp, _vp, _c_i64, _vp, _vp, _vp, _sz, _vp]),
    "gpt_forward_timed": (_c_int, [_CFG, _vp, _vp, _c_int, _c_int, _vp, _vp, _c_i64, _vp, _vp, _vp, _sz, _vp,
                                   _vp, _vp, _c_int]),
    "gpt_status_string": (ctypes.c_char_p, [_c_int]),
    "gpt_debug_layernorm": (_c_int, [_CFG, _vp, _vp, _vp, _c_int, _vp, _vp]),
    "gpt_debug_linear": (_c_int, [_CFG, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
    "gpt_debug_attention": (_c_int, [_CFG, _vp, _vp, _vp, _c_int, _c_int, _vp, _vp]),
    "gpt_debug_attention_rows": (_c_int, [_CFG, _vp, _c_int, _c_int, _vp, _vp]),
    "gpt_decode_workspace_bytes": (_c_int, [_CFG, _c_int, _c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "gpt_prefill": (_c_int, [_CFG, _vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gpt_decode_step": (_c_int, [_CFG, _vp, _vp, _c_int, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _sz, _vp]),
    "gpt_decode_step_noalloc": (_c_int, [_CFG, _vp, _vp, _c_int, _vp, _vp, _vp, _c_int, _vp, _vp, _vp]),
    "gpt_sample": (_c_int, [_CFG, _vp, _c_int, ctypes.POINTER(gpt_sampling), _vp, _vp, _vp, _vp]),
    "gpt_mark_seen": (_c_int, [_CFG, _vp, _c_int, _c_int, _vp, _vp]),
    "gpt_head_backward_workspace_bytes": (_c_int, [_CFG, _c_int, _c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "gpt_head_backward": (_c_int, [_CFG, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gpt_embedding_backward": (_c_int, [_CFG, _vp, _c_int, _c_int, _vp, _vp, _vp]),
    "gpt_forward_train": (_c_int, [_CFG, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gpt_block_backward_workspace_bytes": (_c_int, [_CFG, _c_int, _c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "gpt_block_backward": (_c_int, [_CFG, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
}

_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # torch ships its own HIP runtime; importing it first makes the library
    # bind to that same runtime (one HIP runtime per process, shared streams)
    import torch  # noqa: F401
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m decoder_only_transformer_attn_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


class GPTError(RuntimeError):
    pass


def check(status: int) -> None:
    if status != GPT_OK:
        msg = load().gpt_status_string(status).decode()
        raise GPTError(f"{STATUS.get(status, status)}: {msg}")


def cfg_c(cfg) -> gpt_config:
    return gpt_config(cfg.vocab, cfg.ctx, cfg.n_embd, cfg.n_head, cfg.n_layer, cfg.n_ff, cfg.ln_eps, cfg.dtype,
                      getattr(cfg, "act", 0), getattr(cfg, "post_ln", 0), getattr(cfg, "untied", 0),
                      getattr(cfg, "arch", 0), getattr(cfg, "n_kv_head", 0), getattr(cfg, "rope_theta", 10000.0),
                      getattr(cfg, "alibi", 0))


def param_count(cfg) -> int:
    return int(load().gpt_param_count(ctypes.byref(cfg_c(cfg))))


def param_offsets(cfg):
    if getattr(cfg, "arch", 0) == 1:
        n = 1 + 6 * cfg.n_layer + 1 + (1 if getattr(cfg, "untied", 0) else 0) + 1
    else:
        n = 2 + 12 * cfg.n_layer + (0 if getattr(cfg, "post_ln", 0) else 2) + (1 if getattr(cfg, "untied", 0) else 0) + 1
    arr = (ctypes.c_int64 * n)()
    check(load().gpt_param_offsets(ctypes.byref(cfg_c(cfg)), arr, n))
    return list(arr)


def workspace_bytes(cfg, B: int, T: int) -> int:
    out = ctypes.c_size_t(0)
    check(load().gpt_workspace_bytes(ctypes.byref(cfg_c(cfg)), B, T, ctypes.byref(out)))
    return int(out.value)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def forward(cfg, params, idx, targets=None, logits=None, token_loss=None, mean_loss=None, ws=None,
            stream=None) -> None:
    """Enqueue gpt_forward on the stream.  All tensors are CUDA (HIP) tensors:
    params [param_count] (float32 or bf16), idx int32 [B,T], optional targets
    int32 [B,T], logits [B,T,V] (rows may be further apart than V: a view of
    [B,T,ld] storage goes to gpt_forward_ld), token_loss f32 [B,T], mean_loss
    f32 [1], ws uint8."""
    B, T = idx.shape
    check(load().gpt_forward_ld(ctypes.byref(cfg_c(cfg)), _ptr(params), _ptr(idx), B, T, _ptr(targets),
                                _ptr(logits), _logits_ld(logits, cfg), _ptr(token_loss), _ptr(mean_loss), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream)))


def _logits_ld(logits, cfg) -> int:
    """Row stride of a logits tensor [..., V] whose rows are contiguous and
    evenly spaced (0 when there is none)."""
    if logits is None:
        return 0
    if logits.stride(-1) != 1 or logits.shape[-1] != cfg.vocab:
        raise ValueError("logits rows must be [..., V] with unit column stride")
    ld = logits.stride(-2) if logits.dim() >= 2 else cfg.vocab
    if logits.dim() == 3 and logits.stride(0) != logits.shape[1] * ld:
        raise ValueError("logits rows must be evenly spaced")
    return ld


def head_backward_workspace_bytes(cfg, B: int, T: int) -> int:
    out = ctypes.c_size_t(0)
    check(load().gpt_head_backward_workspace_bytes(ctypes.byref(cfg_c(cfg)), B, T, ctypes.byref(out)))
    return int(out.value)


def head_backward(cfg, params, idx, x, dx, grads, targets=None, mean_loss=None, ws=None, stream=None) -> None:
    """Enqueue gpt_head_backward: x f32 [B*T, C] (rows the final LayerNorm
    reads, or the final hidden rows of a post-LN model), dx f32 [B*T, C]
    (written), grads f32 [param_count] (accumulated), idx / targets int32
    [B, T], mean_loss f32 [1], ws uint8."""
    B, T = idx.shape
    check(load().gpt_head_backward(ctypes.byref(cfg_c(cfg)), _ptr(params), _ptr(idx), B, T, _ptr(targets), _ptr(x),
                                   _ptr(dx), _ptr(grads), _ptr(mean_loss), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(stream)))


def embedding_backward(cfg, idx, dx0, grads, stream=None) -> None:
    """Enqueue gpt_embedding_backward: idx int32 [B, T], dx0 f32 [B*T, C],
    grads f32 [param_count] (token and position rows accumulated)."""
    B, T = idx.shape
    check(load().gpt_embedding_backward(ctypes.byref(cfg_c(cfg)), _ptr(idx), B, T, _ptr(dx0), _ptr(grads),
                                        _stream(stream)))


def forward_train(cfg, params, idx, xs, ws, targets=None, mean_loss=None, stream=None) -> None:
    """Enqueue gpt_forward_train: xs f32 [L+1, B*T, C] receives each block's
    input residual (and ln_f's input); ws as for forward()."""
    B, T = idx.shape
    check(load().gpt_forward_train(ctypes.byref(cfg_c(cfg)), _ptr(params), _ptr(idx), B, T, _ptr(targets), _ptr(xs),
                                   _ptr(mean_loss), _ptr(ws), ws.numel(), _stream(stream)))


def block_backward_workspace_bytes(cfg, B: int, T: int) -> int:
    out = ctypes.c_size_t(0)
    check(load().gpt_block_backward_workspace_bytes(ctypes.byref(cfg_c(cfg)), B, T, ctypes.byref(out)))
    return int(out.value)


def block_backward(cfg, params, layer: int, B: int, T: int, x, dy, dx, grads, ws, stream=None) -> None:
    """Enqueue gpt_block_backward for block `layer`: x, dy, dx f32 [B*T, C];
    grads f32 [param_count] (accumulated)."""
    check(load().gpt_block_backward(ctypes.byref(cfg_c(cfg)), _ptr(params), layer, B, T, _ptr(x), _ptr(dy), _ptr(dx),
                                    _ptr(grads), _ptr(ws), ws.numel(), _stream(stream)))


def gradients(cfg, params, idx, grads, targets=None, stream=None):
    """Every parameter gradient of the mean next-token loss (pre-LN GPT-2
    blocks), accumulated into grads: training forward, head backward, the
    blocks in reverse, embedding backward.  Returns the mean loss tensor."""
    import torch
    B, T = idx.shape
    M, C, L = B * T, cfg.n_embd, cfg.n_layer
    dev = idx.device
    xs = torch.empty((L + 1, M, C), dtype=torch.float32, device=dev)
    loss = torch.zeros(1, dtype=torch.float32, device=dev)
    ws = torch.empty(max(workspace_bytes(cfg, B, T), head_backward_workspace_bytes(cfg, B, T),
                         block_backward_workspace_bytes(cfg, B, T) if L else 0), dtype=torch.uint8, device=dev)
    forward_train(cfg, params, idx, xs, ws, targets, None, stream)   # residual streams only
    d = torch.empty((M, C), dtype=torch.float32, device=dev)
    d2 = torch.empty_like(d)
    head_backward(cfg, params, idx, xs[L], d, grads, targets, loss, ws, stream)   # (the loss is computed here)
    for l in range(L - 1, -1, -1):
        block_backward(cfg, params, l, B, T, xs[l], d, d2, grads, ws, stream)
        d, d2 = d2, d
    embedding_backward(cfg, idx, d, grads, stream)
    return loss


KERNEL = {"head": 0, "qkv": 1, "attn": 2, "proj": 3, "fc": 4, "fcproj": 5, "ln": 6}


def forward_timed(cfg, params, idx, targets, logits, token_loss, mean_loss, ws, ev_begin: int, ev_end: int,
                  which: str, stream=None) -> None:
    """gpt_forward with hipEvent_t handles recorded around one kernel class."""
    B, T = idx.shape
    check(load().gpt_forward_timed(ctypes.byref(cfg_c(cfg)), _ptr(params), _ptr(idx), B, T, _ptr(targets),
                                   _ptr(logits), _logits_ld(logits, cfg), _ptr(token_loss), _ptr(mean_loss), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream), ev_begin, ev_end,
                                   KERNEL[which]))


class HipEvents:
    """Raw hipEvent_t handles from libamdhip64 (torch's Event does not expose its handle)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def elapsed_ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)
        self.ev = []


def torch_dtype(cfg):
    import torch
    return torch.bfloat16 if cfg.dtype == 1 else torch.float32


def params_to_device(cfg, blob, device="cuda"):
    """Upload a packed blob (float32 array, or uint16 bf16 bits) as a device tensor of the config dtype."""
    import numpy as np
    import torch
    if cfg.dtype == 1:
        t = torch.from_numpy(np.ascontiguousarray(blob).view(np.int16)).to(device)
        return t.view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(blob, dtype=np.float32)).to(device)


def _poison(t) -> None:
    """Every byte of t set to 0xFF (a NaN in bf16 and fp32)."""
    t.view(-1).view(__import__("torch").uint8).fill_(255)


class Forward:
    """Holds the output and workspace tensors for repeated gpt_forward calls on one shape."""

    def __init__(self, cfg, B: int, T: int, want_logits: bool = True, device="cuda", poison: bool = False,
                 logits_ld: int = 0):
        """poison: fill the workspace and the outputs with 0xFF bytes (NaN in
        bf16 and fp32), so that a read of anything the call did not write
        first shows up in the results.  logits_ld: row stride of the logits
        storage (>= V; 0 = V); self.logits is then the [B, T, V] view of
        [B, T, logits_ld] storage, kept in self.logits_storage."""
        import torch
        self.cfg, self.B, self.T = cfg, B, T
        self.ws = torch.empty(workspace_bytes(cfg, B, T), dtype=torch.uint8, device=device)
        ld = logits_ld or cfg.vocab
        self.logits_storage = (torch.empty((B, T, ld), dtype=torch_dtype(cfg), device=device) if want_logits
                               else None)
        self.logits = self.logits_storage[..., :cfg.vocab] if want_logits else None
        self.token_loss = torch.empty((B, T), dtype=torch.float32, device=device)
        self.mean_loss = torch.empty((1,), dtype=torch.float32, device=device)
        if poison:
            for t in (self.ws, self.logits_storage, self.token_loss, self.mean_loss):
                if t is not None:
                    _poison(t)

    def __call__(self, params, idx, targets=None, stream=None):
        forward(self.cfg, params, idx, targets, self.logits, self.token_loss, self.mean_loss, self.ws, stream)
        return self.logits, self.token_loss, self.mean_loss


def decode_workspace_bytes(cfg, B: int, Tp: int) -> int:
    out = ctypes.c_size_t(0)
    check(load().gpt_decode_workspace_bytes(ctypes.byref(cfg_c(cfg)), B, Tp, ctypes.byref(out)))
    return int(out.value)


def prefill(cfg, params, idx, k_cache, v_cache, pos, next_tok, last_logits=None, ws=None, stream=None) -> None:
    """Enqueue gpt_prefill.  idx int32 [B, Tp]; caches [L, B, H, Tmax, D]; pos int32 [1]; next_tok int32 [B]."""
    B, Tp = idx.shape
    Tmax = k_cache.shape[3] if k_cache.dim() == 5 else 0
    check(load().gpt_prefill(ctypes.byref(cfg_c(cfg)), _ptr(params), _ptr(idx), B, Tp, _ptr(k_cache), _ptr(v_cache),
                             Tmax, _ptr(pos), _ptr(next_tok), _ptr(last_logits), _ptr(ws),
                             0 if ws is None else ws.numel(), _stream(stream)))


def decode_step(cfg, params, tok, k_cache, v_cache, pos, next_tok, logits=None, ws=None, stream=None) -> None:
    """Enqueue gpt_decode_step.  tok, next_tok int32 [B] (may be the same tensor)."""
    B = tok.shape[0]
    Tmax = k_cache.shape[3] if k_cache.dim() == 5 else 0
    check(load().gpt_decode_step(ctypes.byref(cfg_c(cfg)), _ptr(params), _ptr(tok), B, _ptr(pos), _ptr(k_cache),
                                 _ptr(v_cache), Tmax, _ptr(next_tok), _ptr(logits), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(stream)))


def decode_step_noalloc(cfg, params, tok, k_cache, v_cache, pos, next_tok, logits=None, stream=None) -> None:
    """Enqueue gpt_decode_step_noalloc (the workspace is the library's static
    per-GPU array; calls on one GPU must not overlap)."""
    B = tok.shape[0]
    Tmax = k_cache.shape[3] if k_cache.dim() == 5 else 0
    check(load().gpt_decode_step_noalloc(ctypes.byref(cfg_c(cfg)), _ptr(params), _ptr(tok), B, _ptr(pos),
                                         _ptr(k_cache), _ptr(v_cache), Tmax, _ptr(next_tok), _ptr(logits),
                                         _stream(stream)))


def sampling(temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0, repetition_penalty: float = 1.0):
    return gpt_sampling(float(temperature), int(top_k), float(top_p), float(repetition_penalty))


def seen_words(cfg) -> int:
    return (cfg.vocab + 31) // 32


def sample(cfg, logits, s, u=None, seen=None, next_tok=None, stream=None):
    """Enqueue gpt_sample.  logits [B, V] (compute dtype); s = sampling(...);
    u float32 [B] uniforms in [0, 1); seen int32 [B, seen_words(cfg)] bit sets
    (or None); next_tok int32 [B] (allocated if None).  Returns next_tok."""
    import torch
    B = logits.shape[0]
    if next_tok is None:
        next_tok = torch.empty((B,), dtype=torch.int32, device=logits.device)
    check(load().gpt_sample(ctypes.byref(cfg_c(cfg)), _ptr(logits), B, ctypes.byref(s), _ptr(u), _ptr(seen),
                            _ptr(next_tok), _stream(stream)))
    return next_tok


def mark_seen(cfg, tokens, seen, stream=None) -> None:
    """Enqueue gpt_mark_seen: the bits of tokens int32 [B, T] set in seen."""
    B, T = tokens.shape
    check(load().gpt_mark_seen(ctypes.byref(cfg_c(cfg)), _ptr(tokens), B, T, _ptr(seen), _stream(stream)))


class Decoder:
    """Caches, position counter and workspace for decoding B sequences with
    prompts of Tp tokens and at most Tmax cached positions: greedy by
    default, or sampled (prefill / step with `sampling=` and one uniform per
    sequence in `u`; a repetition penalty reads and updates self.seen)."""

    def __init__(self, cfg, B: int, Tp: int, Tmax: int, device="cuda", poison: bool = False):
        """poison: fill the workspace and both caches with 0xFF bytes (NaN):
        cache positions past the current one are never read, and nothing in
        the workspace is read before the call writes it."""
        import torch
        H = cfg.n_head
        D = cfg.n_embd // H
        Hkv = getattr(cfg, "n_kv_head", 0) or H     # caches hold the K/V heads only
        self.cfg, self.B, self.Tp, self.Tmax = cfg, B, Tp, Tmax
        shape = (max(cfg.n_layer, 1), B, Hkv, Tmax, D)
        self.k_cache = torch.zeros(shape, dtype=torch_dtype(cfg), device=device)
        self.v_cache = torch.zeros(shape, dtype=torch_dtype(cfg), device=device)
        self.pos = torch.zeros((1,), dtype=torch.int32, device=device)
        self.tok = torch.zeros((B,), dtype=torch.int32, device=device)
        self.ws = torch.empty(decode_workspace_bytes(cfg, B, Tp), dtype=torch.uint8, device=device)
        self.seen = torch.zeros((B, seen_words(cfg)), dtype=torch.int32, device=device)
        self._logits = None
        if poison:
            for t in (self.ws, self.k_cache, self.v_cache):
                _poison(t)

    def _row_logits(self, logits):
        import torch
        if logits is not None:
            return logits
        if self._logits is None:
            self._logits = torch.empty((self.B, self.cfg.vocab), dtype=torch_dtype(self.cfg), device=self.tok.device)
        return self._logits

    def prefill(self, params, idx, last_logits=None, stream=None, sampling=None, u=None):
        if sampling is None:
            prefill(self.cfg, params, idx, self.k_cache, self.v_cache, self.pos, self.tok, last_logits, self.ws,
                    stream)
            return self.tok
        z = self._row_logits(last_logits)
        prefill(self.cfg, params, idx, self.k_cache, self.v_cache, self.pos, self.tok, z, self.ws, stream)
        mark_seen(self.cfg, idx, self.seen, stream)
        return sample(self.cfg, z, sampling, u, self.seen, self.tok, stream)

    def step(self, params, logits=None, stream=None, sampling=None, u=None):
        """Feed the last chosen tokens; self.tok is overwritten with the next ones."""
        if sampling is None:
            decode_step(self.cfg, params, self.tok, self.k_cache, self.v_cache, self.pos, self.tok, logits, self.ws,
                        stream)
            return self.tok
        z = self._row_logits(logits)
        decode_step(self.cfg, params, self.tok, self.k_cache, self.v_cache, self.pos, self.tok, z, self.ws, stream)
        return sample(self.cfg, z, sampling, u, self.seen, self.tok, stream)


def debug_layernorm(cfg, x, g, b, out, stream=None) -> None:
    check(load().gpt_debug_layernorm(ctypes.byref(cfg_c(cfg)), _ptr(x), _ptr(g), _ptr(b), x.shape[0], _ptr(out),
                                     _stream(stream)))


def debug_linear(cfg, A, W, bias, out, act=0, out_f32=False, stream=None) -> None:
    M, K = A.shape
    N = W.shape[0]
    check(load().gpt_debug_linear(ctypes.byref(cfg_c(cfg)), _ptr(A), _ptr(W), _ptr(bias), M, N, K, act,
                                  1 if out_f32 else 0, _ptr(out), _stream(stream)))


def debug_attention(cfg, q, k, u, out, stream=None) -> None:
    """q, k, u: [B, H, T, D] device tensors; out [B*T, C]."""
    B, H, T, D = q.shape
    check(load().gpt_debug_attention(ctypes.byref(cfg_c(cfg)), _ptr(q), _ptr(k), _ptr(u), B, T, _ptr(out),
                                     _stream(stream)))


def debug_attention_rows(cfg, qkv, B: int, T: int, out, stream=None) -> None:
    """qkv: [B*T, 3C] token-major q | k | u rows (the forward's c_attn output); out [B*T, C]."""
    check(load().gpt_debug_attention_rows(ctypes.byref(cfg_c(cfg)), _ptr(qkv), B, T, _ptr(out), _stream(stream)))
