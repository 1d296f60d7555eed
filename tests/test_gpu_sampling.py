"""GPU parity of the sampler (gpt_sample through the C ABI) against the
sampling oracle on the same logits, seen sets and uniforms.

Both sides rank identical float32 weights (exp in float64 rounded once) and
decide on float64 masses, so the chosen tokens must be equal, bit for bit
(a difference needs a uniform or p * Z within about 1e-15 of a boundary).
Logit rows cover flat and peaked distributions, many ties (integer logits),
ragged vocabularies and the full GPT-2 vocabulary; settings cover greedy,
plain temperature, top-k, top-p, their combination and the repetition
penalty (the ids of a 64-row batch exercise every path at once).
"""
import numpy as np
import pytest

from decoder_only_transformer_attn_amd import synth
from oracle import sampling_oracle as S

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lib():
    from decoder_only_transformer_attn_amd import lib
    lib.load()
    return lib


def _bits(seen_bool):
    """[B, V] bool -> [B, ceil(V/32)] int32 bit sets."""
    B, V = seen_bool.shape
    W = (V + 31) // 32
    out = np.zeros((B, W), dtype=np.uint32)
    for b in range(B):
        idx = np.nonzero(seen_bool[b])[0]
        np.bitwise_or.at(out[b], idx >> 5, (np.uint32(1) << (idx & 31).astype(np.uint32)))
    return out.view(np.int32)


def _unbits(words, V):
    w = words.view(np.uint32)
    i = np.arange(V)
    return ((w[:, i >> 5] >> (i & 31).astype(np.uint32)) & 1).astype(bool)


SETTINGS = [  # temperature, top_k, top_p, penalty
    (0.0, 0, 1.0, 1.0), (1.0, 0, 1.0, 1.0), (0.8, 50, 1.0, 1.0), (0.7, 0, 0.9, 1.0),
    (1.3, 200, 0.95, 1.1), (0.5, 1, 1.0, 1.0), (1.0, 0, 0.3, 1.3), (0.0, 0, 1.0, 1.4), (2.0, 7, 0.5, 1.0)]


def _rows(V, B, kind, rng):
    if kind == "flat":
        z = rng.normal(0, 0.3, (B, V))
    elif kind == "peaked":
        z = rng.normal(0, 3.0, (B, V))
    else:   # ties: few distinct values
        z = rng.integers(-3, 3, (B, V)).astype(np.float64)
    return z.astype(np.float32)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("V,B", [(50257, 64), (257, 5), (17, 3), (1, 2), (1025, 4)])
@pytest.mark.parametrize("kind", ["flat", "peaked", "ties"])
def test_sampler_matches_oracle(dtype, V, B, kind):
    lib = _lib()
    cfg = synth.GPTConfig(vocab=V, ctx=8, n_embd=16, n_head=2, n_layer=1, n_ff=64, dtype=dtype)
    rng = np.random.default_rng(V * 31 + B + len(kind))
    z = _rows(V, B, kind, rng)
    td = lib.torch_dtype(cfg)
    zt = torch.from_numpy(z).to(td).cuda()
    zin = zt.float().cpu().numpy()                      # the values the kernel reads (bf16-rounded)
    seen0 = rng.random((B, V)) < 0.2
    for (t, k, p, a) in SETTINGS:
        u = rng.random(B).astype(np.float32)
        seen = torch.from_numpy(_bits(seen0)).cuda()
        got = lib.sample(cfg, zt, lib.sampling(t, k, p, a), torch.from_numpy(u).cuda(), seen)
        torch.cuda.synchronize()
        ref = S.sample_rows(zin, seen0, t, k, p, a, u)
        np.testing.assert_array_equal(got.cpu().numpy(), ref, err_msg=f"settings {(t, k, p, a)}")
        # the chosen tokens' bits are set, the others unchanged
        after = _unbits(seen.cpu().numpy(), V)
        expect = seen0.copy()
        expect[np.arange(B), ref] = True
        np.testing.assert_array_equal(after, expect)


def test_sampler_without_seen_and_determinism():
    lib = _lib()
    cfg = synth.GPTConfig(vocab=50257, ctx=8, n_embd=16, n_head=2, n_layer=1, n_ff=64, dtype=synth.BF16)
    rng = np.random.default_rng(11)
    zt = torch.from_numpy(_rows(50257, 64, "flat", rng)).to(torch.bfloat16).cuda()
    u = torch.from_numpy(rng.random(64).astype(np.float32)).cuda()
    s = lib.sampling(0.9, 0, 0.92, 1.2)                # a penalty without a seen set has no effect
    a = lib.sample(cfg, zt, s, u).cpu().numpy()
    b = lib.sample(cfg, zt, s, u).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    ref = S.sample_rows(zt.float().cpu().numpy(), None, 0.9, 0, 0.92, 1.2, u.cpu().numpy())
    np.testing.assert_array_equal(a, ref)


def test_stratified_draws_follow_the_filtered_distribution():
    # one row repeated with a stratified set of uniforms: the token frequencies
    # are the renormalised top-k / top-p probabilities within 2 / N
    lib = _lib()
    V, N = 40, 4096
    cfg = synth.GPTConfig(vocab=V, ctx=8, n_embd=16, n_head=2, n_layer=1, n_ff=64, dtype=synth.F32)
    z = np.random.default_rng(2).normal(0, 1.5, V).astype(np.float32)
    zt = torch.from_numpy(np.tile(z, (N, 1))).cuda()
    u = torch.from_numpy(((np.arange(N) + 0.5) / N).astype(np.float32)).cuda()
    got = lib.sample(cfg, zt, lib.sampling(0.9, 10, 0.8), u).cpu().numpy()
    cand, w = S.filtered(z, None, 0.9, 10, 0.8)
    expect = np.zeros(V)
    expect[cand] = w / w.sum()
    assert np.all(np.abs(np.bincount(got, minlength=V) / N - expect) <= 2.0 / N)


def test_mark_seen_sets_bits():
    lib = _lib()
    cfg = synth.GPTConfig(vocab=300, ctx=8, n_embd=16, n_head=2, n_layer=1, n_ff=64, dtype=synth.BF16)
    rng = np.random.default_rng(4)
    toks = rng.integers(0, 300, (3, 17)).astype(np.int32)
    toks[1, 3] = -1                                    # ignored
    seen = torch.zeros((3, 10), dtype=torch.int32, device="cuda")
    seen[2, 0] = 1                                     # token 0 of row 2 already set
    lib.mark_seen(cfg, torch.from_numpy(toks).cuda(), seen)
    got = _unbits(seen.cpu().numpy(), 300)
    expect = np.zeros((3, 300), bool)
    for b in range(3):
        expect[b, toks[b][toks[b] >= 0]] = True
    expect[2, 0] = True
    np.testing.assert_array_equal(got, expect)


def test_sampled_decode_follows_the_oracle_sampler():
    # prefill + steps with sampling: every emitted token is the oracle's draw
    # from the GPU's own logits of that step, the seen set the prompt plus the
    # tokens drawn so far
    lib = _lib()
    cfg = synth.GPTConfig(vocab=257, ctx=64, n_embd=64, n_head=2, n_layer=2, n_ff=256, dtype=synth.BF16)
    params = synth.make_params(cfg, seed=7, cfg_id=9, init="stress")
    B, Tp, steps = 6, 9, 8
    prompt = synth.make_ids(cfg, B, Tp, seed=7, cfg_id=9)
    P = lib.params_to_device(cfg, synth.pack(cfg, params))
    dec = lib.Decoder(cfg, B, Tp, 32)
    s = lib.sampling(0.9, 40, 0.9, 1.2)
    rng = np.random.default_rng(1)
    z = torch.empty((B, cfg.vocab), dtype=torch.bfloat16, device="cuda")
    seen = np.zeros((B, cfg.vocab), bool)
    for b in range(B):
        seen[b, prompt[b]] = True
    for it in range(steps + 1):
        u = rng.random(B).astype(np.float32)
        if it == 0:
            tok = dec.prefill(P, torch.from_numpy(prompt).cuda(), last_logits=z, sampling=s,
                              u=torch.from_numpy(u).cuda())
        else:
            tok = dec.step(P, logits=z, sampling=s, u=torch.from_numpy(u).cuda())
        torch.cuda.synchronize()
        ref = S.sample_rows(z.float().cpu().numpy(), seen, 0.9, 40, 0.9, 1.2, u)
        np.testing.assert_array_equal(tok.cpu().numpy(), ref, err_msg=f"emission {it}")
        seen[np.arange(B), ref] = True
    assert int(dec.pos.item()) == Tp + steps
