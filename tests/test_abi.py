"""C-ABI checks that run without a GPU: the library loads, exports every
symbol that include/gptmi.h declares, and its host-only logic (parameter
count and offsets, workspace plan, argument validation) behaves as
documented.  Validation happens before any HIP call, so dummy host pointers
are safe here."""
import ctypes
import os
import re

import pytest

from decoder_only_transformer_attn_amd import lib, synth
from oracle import gpt_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptmi.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gpt_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = lib.load()
    names = _declared_functions()
    assert "gpt_forward" in names and "gpt_param_count" in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in gptmi.h but not exported"
    assert set(names) == set(lib.SIGNATURES), "binding and header disagree"


@pytest.mark.parametrize("cfg", [synth.MICRO, synth.MINI, synth.GPT2])
def test_param_count_and_offsets_match_packing(cfg):
    assert lib.param_count(cfg) == O.param_count(cfg.vocab, cfg.n_embd, cfg.n_layer, cfg.ctx, cfg.n_ff)
    offs = lib.param_offsets(cfg)
    layout = synth.blob_layout(cfg)
    assert offs == [off for _, _, off in layout]


def test_gpt2_param_count_printed_value():
    # 第 25 章 从小 GPT 到 GPT-2, §25.4
    assert lib.param_count(synth.GPT2) == 124439808
    assert lib.param_count(synth.MICRO) == 7056


def _fwd(cfg, B=2, T=4, params=1, idx=1, ws=1, ws_bytes=1 << 30, cfg_ptr=True):
    L = lib.load()
    c = lib.cfg_c(cfg)
    return L.gpt_forward(ctypes.byref(c) if cfg_ptr else None, params, idx, B, T, None, None, None, None,
                         ws, ws_bytes, None)


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


# These calls pass dummy host pointers and rely on validation failing before
# any HIP call; they run only where no GPU is visible.
@pytest.mark.skipif(not _no_gpu(), reason="dummy-pointer validation tests run only without a GPU")
def test_forward_validation_before_any_hip_call():
    import dataclasses as dc
    m = synth.MICRO
    assert _fwd(m, cfg_ptr=False) == -1
    assert _fwd(m, params=None) == -1
    assert _fwd(m, idx=None) == -1
    assert _fwd(m, ws=None) == -1
    assert _fwd(dc.replace(m, n_head=3)) == -2                     # C % H != 0 (Day 16 三十八)
    assert _fwd(dc.replace(m, n_embd=12, n_head=2)) == -2          # C not a multiple of 4/8
    assert _fwd(dc.replace(synth.GPT2, n_head=192)) == -2         # bf16 needs D % 8 == 0 (D = 4)
    assert _fwd(dc.replace(synth.GPT2, n_head=3)) == -2           # D = 256 > 128
    assert _fwd(dc.replace(m, dtype=7)) == -6
    assert _fwd(dc.replace(m, vocab=0)) == -2
    assert _fwd(m, T=13) == -3                                     # T > ctx (Day 16 三十九)
    assert _fwd(m, B=0) == -4
    assert _fwd(m, T=0) == -4
    assert _fwd(m, ws_bytes=16) == -5
    msg = lib.load().gpt_status_string(-3).decode()
    assert "context" in msg
    # gpt_forward_ld: a logits row stride below V (0 means V) or past 2^31
    L = lib.load()
    c = lib.cfg_c(m)
    for ld, want in [(m.vocab - 1, -4), (1 << 32, -4), (-5, -4)]:
        assert L.gpt_forward_ld(ctypes.byref(c), 1, 1, 2, 4, None, None, ld, None, None, 1, 1 << 30, None) == want
    assert L.gpt_forward_ld(ctypes.byref(c), None, 1, 2, 4, None, None, m.vocab + 3, None, None, 1, 1 << 30,
                            None) == -1


@pytest.mark.skipif(not _no_gpu(), reason="dummy-pointer validation tests run only without a GPU")
def test_debug_entry_validation():
    L = lib.load()
    c = lib.cfg_c(synth.MICRO)
    assert L.gpt_debug_linear(ctypes.byref(c), 1, 1, None, 4, 4, 6, 0, 0, 1, None) == -4  # K % 4
    assert L.gpt_debug_linear(ctypes.byref(c), None, 1, None, 4, 4, 8, 0, 0, 1, None) == -1
    assert L.gpt_debug_layernorm(ctypes.byref(c), 1, 1, 1, 0, 1, None) == -4
    assert L.gpt_debug_attention(ctypes.byref(c), 1, 1, 1, 0, 12, 1, None) == -4  # B = 0
    assert L.gpt_debug_attention_rows(ctypes.byref(c), 1, 2, 0, 1, None) == -4    # T = 0
    assert L.gpt_debug_attention_rows(ctypes.byref(c), None, 2, 12, 1, None) == -1


def test_workspace_grows_with_batch():
    a = lib.workspace_bytes(synth.GPT2, 8, 1024)
    b = lib.workspace_bytes(synth.GPT2, 32, 1024)
    assert 3.5 * a < b < 4.5 * a
    with pytest.raises(lib.GPTError):
        lib.workspace_bytes(synth.GPT2, 1, 1025)


@pytest.mark.skipif(not _no_gpu(), reason="dummy-pointer validation tests run only without a GPU")
def test_decode_validation_before_any_hip_call():
    L = lib.load()
    m = synth.MICRO                                   # ctx 12
    c = ctypes.byref(lib.cfg_c(m))
    big = 1 << 30

    def pre(B=2, Tp=4, kc=1, vc=1, Tmax=12, pos=1, nt=1, ws=1, ws_bytes=big, idx=1):
        return L.gpt_prefill(c, 1, idx, B, Tp, kc, vc, Tmax, pos, nt, None, ws, ws_bytes, None)

    def step(B=2, kc=1, vc=1, Tmax=12, pos=1, nt=1, tok=1, ws=1, ws_bytes=big):
        return L.gpt_decode_step(c, 1, tok, B, pos, kc, vc, Tmax, nt, None, ws, ws_bytes, None)

    assert pre(kc=None) == -1 and pre(pos=None) == -1 and pre(nt=None) == -1 and pre(idx=None) == -1
    assert pre(Tmax=13) == -4                         # cache longer than the position table
    assert pre(Tmax=0) == -4 and pre(B=0) == -4 and pre(Tp=0) == -4
    assert pre(Tp=5, Tmax=4) == -3                    # prompt longer than the cache
    assert pre(ws_bytes=16) == -5
    assert step(vc=None) == -1 and step(tok=None) == -1 and step(pos=None) == -1
    assert step(Tmax=13) == -4 and step(B=0) == -4
    assert step(ws_bytes=16) == -5


def test_decode_workspace_covers_step_and_is_smaller_than_forward():
    pre = lib.decode_workspace_bytes(synth.GPT2, 64, 128)
    assert pre < lib.workspace_bytes(synth.GPT2, 64, 128)   # no K/U copies, head on B rows only
    assert lib.decode_workspace_bytes(synth.GPT2, 64, 1) <= pre
    with pytest.raises(lib.GPTError):
        lib.decode_workspace_bytes(synth.GPT2, 1, 1025)


@pytest.mark.skipif(not _no_gpu(), reason="dummy-pointer validation tests run only without a GPU")
def test_sample_validation_before_any_hip_call():
    L = lib.load()
    c = ctypes.byref(lib.cfg_c(synth.GPT2))

    def smp(logits=1, B=4, s=None, u=1, seen=None, nt=1, cfg=c):
        s = s if s is not None else lib.sampling(0.8, 50, 0.9, 1.1)
        return L.gpt_sample(cfg, logits, B, ctypes.byref(s), u, seen, nt, None)

    assert smp(logits=None) == -1 and smp(nt=None) == -1
    assert smp(u=None) == -1                                   # a draw needs its uniform
    assert smp(B=0) == -4
    assert smp(s=lib.sampling(float("nan"))) == -4
    assert smp(s=lib.sampling(1.0, 0, 0.0)) == -4              # top-p must be positive
    assert smp(s=lib.sampling(1.0, 0, 1.0, 0.0)) == -4         # penalty must be positive
    big = ctypes.byref(lib.cfg_c(synth.GPTConfig(vocab=60000, ctx=8, n_embd=16, n_head=2, n_layer=1, n_ff=64)))
    assert smp(cfg=big) == -2                                  # vocabulary beyond one block's slices
    assert L.gpt_mark_seen(c, None, 2, 3, 1, None) == -1 and L.gpt_mark_seen(c, 1, 0, 3, 1, None) == -4


@pytest.mark.parametrize("post_ln,untied", [(1, 0), (0, 1), (1, 1)])
def test_param_count_and_offsets_of_variants(post_ln, untied):
    import dataclasses as dc
    cfg = dc.replace(synth.MINI, post_ln=post_ln, untied=untied, act=1)
    assert lib.param_count(cfg) == O.param_count(cfg.vocab, cfg.n_embd, cfg.n_layer, cfg.ctx, cfg.n_ff,
                                                 post_ln=bool(post_ln), untied=bool(untied))
    assert lib.param_offsets(cfg) == [off for _, _, off in synth.blob_layout(cfg)]


def test_variant_flags_are_validated():
    import dataclasses as dc
    for bad in (dict(act=2), dict(post_ln=-1), dict(untied=3)):
        assert lib.load().gpt_param_count(ctypes.byref(lib.cfg_c(dc.replace(synth.MICRO, **bad)))) == -2


def test_backward_validation_and_workspace():
    L = lib.load()
    cfg = synth.MICRO
    c = ctypes.byref(lib.cfg_c(cfg))
    w1 = lib.head_backward_workspace_bytes(cfg, 2, 5)
    w2 = lib.head_backward_workspace_bytes(cfg, 4, 10)
    assert 0 < w1 < w2

    def hb(params=1, idx=1, B=2, T=5, x=1, dx=1, grads=1, ws=1, ws_bytes=1 << 40):
        return L.gpt_head_backward(c, params, idx, B, T, None, x, dx, grads, None, ws, ws_bytes, None)

    for kw in (dict(params=None), dict(idx=None), dict(x=None), dict(dx=None), dict(grads=None), dict(ws=None)):
        assert hb(**kw) == lib.GPT_ERR_NULL, kw
    assert hb(B=0) == lib.GPT_ERR_SHAPE and hb(T=0) == lib.GPT_ERR_SHAPE
    assert hb(B=(1 << 20) // cfg.ctx + 1, T=cfg.ctx) == lib.GPT_ERR_SHAPE    # more than 2^20 rows
    assert hb(T=cfg.ctx + 1) == lib.GPT_ERR_SEQ_TOO_LONG
    assert hb(ws_bytes=w1 - 1) == lib.GPT_ERR_WORKSPACE
    eb = L.gpt_embedding_backward
    assert eb(c, None, 2, 5, 1, 1, None) == lib.GPT_ERR_NULL and eb(c, 1, 2, 5, None, 1, None) == lib.GPT_ERR_NULL
    assert eb(c, 1, 2, 5, 1, None, None) == lib.GPT_ERR_NULL
    assert eb(c, 1, 0, 5, 1, 1, None) == lib.GPT_ERR_SHAPE
    assert eb(c, 1, 2, cfg.ctx + 1, 1, 1, None) == lib.GPT_ERR_SEQ_TOO_LONG


@pytest.mark.parametrize("Hkv,untied,L", [(0, 0, 2), (2, 1, 3), (1, 0, 1), (4, 1, 0)])
def test_llama_param_count_and_offsets(Hkv, untied, L):
    import dataclasses as dc
    from oracle import llama_oracle as LO
    cfg = synth.GPTConfig(vocab=101, ctx=32, n_embd=64, n_head=4, n_layer=L, n_ff=96, arch=1, n_kv_head=Hkv,
                          untied=untied)
    assert lib.param_count(cfg) == LO.param_count(cfg.vocab, cfg.n_embd, L, 4, cfg.kv_heads, cfg.n_ff, bool(untied))
    assert lib.param_count(cfg) == synth.blob_numel(cfg)
    assert lib.param_offsets(cfg) == [off for _, _, off in synth.blob_layout(cfg)]
    bf = dc.replace(cfg, dtype=synth.BF16)
    assert lib.param_count(bf) == synth.blob_numel(bf)


def test_llama_config_is_validated():
    import dataclasses as dc
    good = synth.GPTConfig(vocab=101, ctx=32, n_embd=64, n_head=4, n_layer=1, n_ff=96, arch=1, n_kv_head=2)
    count = lambda c: lib.load().gpt_param_count(ctypes.byref(lib.cfg_c(c)))
    assert count(good) > 0
    for bad in (dict(n_kv_head=3), dict(n_kv_head=8), dict(n_kv_head=-1), dict(act=1), dict(post_ln=1),
                dict(rope_theta=0.0), dict(rope_theta=float("inf")), dict(arch=2)):
        assert count(dc.replace(good, **bad)) == lib.GPT_ERR_CONFIG, bad
    assert count(dc.replace(good, arch=0, n_kv_head=1)) == lib.GPT_ERR_CONFIG   # no grouping in GPT-2 blocks
    assert count(dc.replace(good, alibi=1)) > 0
    assert count(dc.replace(good, alibi=2)) == lib.GPT_ERR_CONFIG
    assert count(dc.replace(good, arch=0, n_kv_head=0, alibi=1)) == lib.GPT_ERR_CONFIG   # LLaMA-style blocks only
    assert count(dc.replace(good, arch=0, n_kv_head=4)) > 0
    # the head backward covers GPT-2 blocks only
    out = ctypes.c_size_t(0)
    assert lib.load().gpt_head_backward_workspace_bytes(ctypes.byref(lib.cfg_c(good)), 2, 4,
                                                        ctypes.byref(out)) == lib.GPT_ERR_CONFIG


def test_block_backward_validation():
    L = lib.load()
    cfg = synth.MICRO
    c = ctypes.byref(lib.cfg_c(cfg))
    w = lib.block_backward_workspace_bytes(cfg, 2, 5)
    assert w > 0

    def bb(layer=0, B=2, T=5, x=1, dy=1, dx=1, grads=1, ws=1, ws_bytes=1 << 40, params=1, cc=c):
        return L.gpt_block_backward(cc, params, layer, B, T, x, dy, dx, grads, ws, ws_bytes, None)

    for kw in (dict(params=None), dict(x=None), dict(dy=None), dict(dx=None), dict(grads=None), dict(ws=None)):
        assert bb(**kw) == lib.GPT_ERR_NULL, kw
    assert bb(layer=-1) == lib.GPT_ERR_SHAPE and bb(layer=cfg.n_layer) == lib.GPT_ERR_SHAPE
    assert bb(B=0) == lib.GPT_ERR_SHAPE and bb(T=cfg.ctx + 1) == lib.GPT_ERR_SEQ_TOO_LONG
    assert bb(ws_bytes=w - 1) == lib.GPT_ERR_WORKSPACE
    import dataclasses as dc
    for var in (dict(post_ln=1), dict(arch=1, n_kv_head=1)):
        bad = ctypes.byref(lib.cfg_c(dc.replace(cfg, **var)))
        assert bb(cc=bad) == lib.GPT_ERR_CONFIG
        assert L.gpt_forward_train(bad, 1, 1, 2, 5, None, 1, None, 1, 1 << 40, None) == lib.GPT_ERR_CONFIG
    assert L.gpt_forward_train(c, 1, 1, 2, 5, None, None, None, 1, 1 << 40, None) == lib.GPT_ERR_NULL


def test_decode_noalloc_validation_before_any_hip_call():
    # every host-checkable condition returns before the scratch lookup (a HIP
    # call, which would fail here without a GPU)
    L = lib.load()
    c = ctypes.byref(lib.cfg_c(synth.GPT2))
    kc = vc = pos = tok = nt = ctypes.c_void_p(16)

    def step(B, Tmax=256, tok_=tok, cfg=c):
        return L.gpt_decode_step_noalloc(cfg, 1, tok_, B, pos, kc, vc, Tmax, nt, None, None)
    assert step(4096) == -5                      # the step's workspace exceeds GPT_DECODE_NOALLOC_BYTES
    assert step(0) == -4 and step(4, Tmax=0) == -4
    assert step(4, tok_=None) == -1
    import dataclasses as dc
    bad = ctypes.byref(lib.cfg_c(dc.replace(synth.GPT2, n_head=5)))
    assert step(4, cfg=bad) == -2
