"""gpt_decode_step_noalloc (no workspace argument: the library's static
per-GPU scratch array) against gpt_decode_step with a caller workspace, on
the same caches, tokens and weights: tokens, logits, caches and the device
position must be identical, bit for bit (the same kernels run on the same
inputs).  Two calls in a row on one GPU, the second with a smaller batch, so
the second call starts on the first call's leftover scratch contents."""
import numpy as np
import pytest

from decoder_only_transformer_attn_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lib():
    from decoder_only_transformer_attn_amd import lib
    lib.load()
    return lib


def _bytes(t):
    return t.contiguous().view(-1).view(torch.uint8)


def _compare(cfg, params, B, Tp, Tmax, steps, seed):
    lib = _lib()
    P = lib.params_to_device(cfg, synth.pack(cfg, params))
    prompt = torch.from_numpy(synth.make_ids(cfg, B, Tp, seed=seed, cfg_id=31)).cuda()
    ref = lib.Decoder(cfg, B, Tp, Tmax, poison=True)
    new = lib.Decoder(cfg, B, Tp, Tmax, poison=True)
    ref.prefill(P, prompt)
    new.prefill(P, prompt)
    td = lib.torch_dtype(cfg)
    for s in range(steps):
        zr = torch.empty((B, cfg.vocab), dtype=td, device="cuda")
        zn = torch.empty((B, cfg.vocab), dtype=td, device="cuda")
        lib.decode_step(cfg, P, ref.tok, ref.k_cache, ref.v_cache, ref.pos, ref.tok, zr, ref.ws)
        lib.decode_step_noalloc(cfg, P, new.tok, new.k_cache, new.v_cache, new.pos, new.tok, zn)
        torch.cuda.synchronize()
        print(f"B={B} step {s}: tokens {new.tok[:6].tolist()}", flush=True)
        assert torch.equal(new.tok, ref.tok), f"step {s}: tokens differ"
        assert torch.equal(_bytes(zn), _bytes(zr)), f"step {s}: logits differ"
    assert torch.equal(_bytes(new.k_cache), _bytes(ref.k_cache))
    assert torch.equal(_bytes(new.v_cache), _bytes(ref.v_cache))
    assert int(new.pos.item()) == int(ref.pos.item()) == Tp + steps


def test_decode_step_noalloc_matches_workspace_step_twice_second_smaller():
    # first call: GPT-2 124M at B = 64 (the split products and their counters
    # in the scratch); second call: a smaller model and batch on the same
    # scratch, which still holds the first call's contents
    cfg = synth.GPT2
    params = synth.make_params(cfg, seed=42, cfg_id=5)
    _compare(cfg, params, 64, 16, 24, 3, seed=1)
    small = synth.GPTConfig(vocab=257, ctx=64, n_embd=64, n_head=2, n_layer=2, n_ff=1536, dtype=synth.BF16)
    _compare(small, synth.make_params(small, seed=6, cfg_id=9, init="stress"), 5, 9, 20, 4, seed=2)
