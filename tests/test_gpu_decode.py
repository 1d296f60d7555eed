"""GPU parity of greedy decoding with the key/value cache (prefill + decode
steps through the C ABI) against the fp64 oracle.

The oracle replays the GPU's own token choices (teacher forcing), so every
step's logits are compared on the same history even where bf16 picks a
different one of several near-tied tokens.  A GPU token is valid if its oracle
logit is within the tie band of the oracle maximum: 1e-4 * max|z| for fp32,
2 * 5e-2 for bf16 (twice the per-logit bound).  Logit bounds are the forward
pass's: fp32 max|dz| <= 1e-4 * max|z_ref|, bf16 max|dz| <= 5e-2.
"""
import dataclasses as dc

import numpy as np
import pytest

from decoder_only_transformer_attn_amd import synth
from oracle import gpt_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lib():
    from decoder_only_transformer_attn_amd import lib
    lib.load()
    return lib


def run_decode(cfg, params, prompt, steps, Tmax, rows=None):
    """Prefill + `steps` decode steps on the GPU.  Returns the emitted tokens
    [B, steps+1], the logits of every emission [B, steps+1, V] (rows `rows`
    only, fp32 numpy) and the final device position."""
    lib = _lib()
    B, Tp = prompt.shape
    P = lib.params_to_device(cfg, synth.pack(cfg, params))
    idx = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    dec = lib.Decoder(cfg, B, Tp, Tmax, poison=True)
    z = torch.empty((steps + 1, B, cfg.vocab), dtype=lib.torch_dtype(cfg), device="cuda")
    toks = torch.empty((steps + 1, B), dtype=torch.int32, device="cuda")
    dec.prefill(P, idx, last_logits=z[0])
    toks[0] = dec.tok
    for s in range(steps):
        dec.step(P, logits=z[s + 1])
        toks[s + 1] = dec.tok
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else list(rows)
    zz = z.float().permute(1, 0, 2)[sel].cpu().numpy()
    return toks.t().cpu().numpy(), zz, int(dec.pos.item()), dec


def check_against_oracle(cfg, params, prompt, toks, z, rows, logit_tol, tie_band):
    P = synth.unpack_f64(cfg, params)
    steps = toks.shape[1] - 1
    sub = prompt[list(rows)]
    ref_tok, ref_z = O.greedy_cached(P, sub, steps, cfg.n_head, cfg.ln_eps, forced=toks[list(rows), :steps])
    for i, b in enumerate(rows):
        err = np.abs(z[i] - ref_z[i]).max()
        print(f"seq {b}: max|dlogit| over {steps + 1} emissions {err:.3e}")
        assert err <= logit_tol(ref_z[i])
        picked = ref_z[i][np.arange(steps + 1), toks[b]]
        assert np.all(picked >= ref_z[i].max(-1) - tie_band(ref_z[i])), "a GPU token is not a greedy choice"
        same = np.mean(toks[b] == ref_tok[i])
        print(f"seq {b}: GPU tokens equal to the oracle's argmax at {same:.3f} of the emissions")


def fp32_tol(zr):
    return 1e-4 * np.abs(zr).max()


@pytest.mark.parametrize("seed,init", [(42, "bench"), (1, "stress"), (3, "stress")])
def test_micro_fp32_decode(seed, init):
    cfg = synth.MICRO                                   # ctx 12: prompt 5 + 7 steps fills it
    params = synth.make_params(cfg, seed=seed, cfg_id=1, init=init)
    prompt = synth.make_ids(cfg, 3, 5, seed=seed, cfg_id=1)
    toks, z, pos, _ = run_decode(cfg, params, prompt, steps=6, Tmax=12)
    assert pos == 11
    check_against_oracle(cfg, params, prompt, toks, z, range(3), fp32_tol, fp32_tol)


@pytest.mark.parametrize("B,Tp,Tmax,steps", [(5, 17, 40, 20), (1, 1, 8, 7), (2, 64, 128, 9), (1, 100, 128, 28)])
def test_minigpt_fp32_decode(B, Tp, Tmax, steps):
    cfg = synth.MINI
    params = synth.make_params(cfg, seed=Tp, cfg_id=2, init="stress")
    prompt = synth.make_ids(cfg, B, Tp, seed=Tp, cfg_id=2)
    toks, z, pos, _ = run_decode(cfg, params, prompt, steps, Tmax)
    assert pos == Tp + steps
    check_against_oracle(cfg, params, prompt, toks, z, range(B), fp32_tol, fp32_tol)


@pytest.mark.parametrize("var", [dict(act=1, post_ln=1, untied=1), dict(post_ln=1), dict(untied=1)],
                         ids=lambda v: "-".join(v))
def test_variant_decode_fp32(var):
    # GPT-1 style blocks (post-LN, no ln_f), exact GELU and an untied head,
    # through prefill and cached steps
    cfg = dc.replace(synth.MINI, **var)
    params = synth.make_params(cfg, seed=9, cfg_id=2, init="stress")
    prompt = synth.make_ids(cfg, 3, 21, seed=9, cfg_id=2)
    toks, z, pos, _ = run_decode(cfg, params, prompt, steps=10, Tmax=40)
    assert pos == 31
    check_against_oracle(cfg, params, prompt, toks, z, range(3), fp32_tol, fp32_tol)


def test_variant_decode_bf16_skinny():
    # the same variants in bf16 at B = 5: skinny products, split-K fc-projection
    cfg = synth.GPTConfig(vocab=300, ctx=64, n_embd=128, n_head=2, n_layer=2, n_ff=1536, dtype=synth.BF16,
                          act=1, post_ln=1, untied=1)
    params = synth.make_params(cfg, seed=10, cfg_id=10, init="stress")
    prompt = synth.make_ids(cfg, 5, 9, seed=10, cfg_id=10)
    toks, z, pos, _ = run_decode(cfg, params, prompt, steps=10, Tmax=32, rows=[0, 4])
    assert pos == 19
    check_against_oracle(cfg, params, prompt, toks, z, [0, 4], bf16_tol, bf16_band)


def test_zero_layer_decode_fp32():
    cfg = dc.replace(synth.MICRO, n_layer=0)
    params = synth.make_params(cfg, seed=3, cfg_id=1, init="stress")
    prompt = synth.make_ids(cfg, 2, 4, seed=3)
    toks, z, pos, _ = run_decode(cfg, params, prompt, steps=3, Tmax=10)
    assert pos == 7
    check_against_oracle(cfg, params, prompt, toks, z, range(2), fp32_tol, fp32_tol)


def test_decode_cache_matches_forward_kv_fp32():
    # after prefill + steps, the cache rows hold the K and U that the oracle's
    # projections give for the same tokens at the same positions
    cfg = synth.MICRO
    params = synth.make_params(cfg, seed=5, cfg_id=1, init="stress")
    prompt = synth.make_ids(cfg, 2, 4, seed=5, cfg_id=1)
    toks, _, pos, dec = run_decode(cfg, params, prompt, steps=3, Tmax=9)
    seq = np.concatenate([prompt, toks[:, :3]], axis=1)               # positions 0..6
    P = synth.unpack_f64(cfg, params)
    kc = dec.k_cache.float().cpu().numpy()
    vc = dec.v_cache.float().cpu().numpy()
    B, T, C, H = 2, 7, cfg.n_embd, cfg.n_head
    x = O.embed(P, seq)
    for l, lp in enumerate(P["layers"]):
        qkv = O.linear(O.layer_norm(x, lp["ln1_g"], lp["ln1_b"], cfg.ln_eps), lp["attn_w"], lp["attn_b"])
        k_ref = qkv[..., C:2 * C].reshape(B, T, H, C // H).transpose(0, 2, 1, 3)
        u_ref = qkv[..., 2 * C:].reshape(B, T, H, C // H).transpose(0, 2, 1, 3)
        x = O.block(x, lp, H, cfg.ln_eps)
        scale = max(np.abs(k_ref).max(), np.abs(u_ref).max())
        assert np.abs(kc[l, :, :, :7] - k_ref).max() <= 1e-4 * scale
        assert np.abs(vc[l, :, :, :7] - u_ref).max() <= 1e-4 * scale
        # rows past the position untouched: still the 0xFF fill of the poisoned caches
        raw = dec.k_cache[l, :, :, 7:].contiguous().view(torch.uint8)
        assert bool((raw == 255).all())


def bf16_tol(_):
    return 5e-2


def bf16_band(_):
    return 1e-1


@pytest.mark.parametrize("B", [3, 70])
def test_small_bf16_decode(B):
    # B <= 64: skinny products and the skinny greedy head; B = 70: tiled paths
    cfg = synth.GPTConfig(vocab=257, ctx=64, n_embd=64, n_head=2, n_layer=2, n_ff=256, dtype=synth.BF16)
    params = synth.make_params(cfg, seed=4, cfg_id=9, init="stress")
    prompt = synth.make_ids(cfg, B, 20, seed=4, cfg_id=9)
    toks, z, pos, _ = run_decode(cfg, params, prompt, steps=12, Tmax=40, rows=[0, 1, B - 1])
    assert pos == 32
    check_against_oracle(cfg, params, prompt, toks, z, [0, 1, B - 1], bf16_tol, bf16_band)


@pytest.mark.parametrize("B", [5, 64])
def test_bf16_decode_split_k(B):
    # n_embd = 128, n_ff = 1536: the step's products are written as K-slices
    # (the fc-projection's K = 1536 in 12), which the attention and the
    # residual LayerNorms add in slice order
    cfg = synth.GPTConfig(vocab=300, ctx=64, n_embd=128, n_head=2, n_layer=2, n_ff=1536, dtype=synth.BF16)
    params = synth.make_params(cfg, seed=8, cfg_id=10, init="stress")
    prompt = synth.make_ids(cfg, B, 9, seed=8, cfg_id=10)
    toks, z, pos, _ = run_decode(cfg, params, prompt, steps=10, Tmax=32, rows=[0, B - 1])
    assert pos == 19
    check_against_oracle(cfg, params, prompt, toks, z, [0, B - 1], bf16_tol, bf16_band)


@pytest.mark.parametrize("B", [5, 64])
def test_bf16_decode_c768(B):
    # GPT-2 widths (C = 768, 12 heads, F = 3072) with one block and a small
    # vocabulary: the step's K-sliced products at their real depths, and the
    # argmax head of at most 64 tokens (B = 5: a partial token tile)
    cfg = dc.replace(synth.GPT2, vocab=1000, n_layer=1)
    params = synth.make_params(cfg, seed=12, cfg_id=12, init="stress")
    prompt = synth.make_ids(cfg, B, 11, seed=12, cfg_id=12)
    toks, z, pos, _ = run_decode(cfg, params, prompt, steps=8, Tmax=24, rows=[0, B - 1])
    assert pos == 19
    check_against_oracle(cfg, params, prompt, toks, z, [0, B - 1], bf16_tol, bf16_band)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_decode_past_256_positions(dtype):
    # a cache longer than one batch of the decode attention (8 keys per group
    # of 32 groups: 256 positions): the steps cross position 256, so the new
    # key is found in the second batch (bf16 at n_embd 128: the K-sliced step,
    # whose new row comes from LDS; fp32: the general step)
    cfg = synth.GPTConfig(vocab=300, ctx=320, n_embd=128, n_head=2, n_layer=2, n_ff=512, dtype=dtype)
    params = synth.make_params(cfg, seed=21, cfg_id=11, init="stress")
    prompt = synth.make_ids(cfg, 3, 250, seed=21, cfg_id=11)
    toks, z, pos, _ = run_decode(cfg, params, prompt, steps=12, Tmax=300, rows=[0, 2])
    assert pos == 262
    tol, band = (fp32_tol, fp32_tol) if dtype == synth.F32 else (bf16_tol, bf16_band)
    check_against_oracle(cfg, params, prompt, toks, z, [0, 2], tol, band)


@pytest.fixture(scope="module")
def gpt2_decode_run():
    cfg = synth.GPT2
    params = synth.make_params(cfg, seed=42, cfg_id=5)
    prompt = synth.make_ids(cfg, 64, 128, seed=42, cfg_id=5)
    toks, z, pos, dec = run_decode(cfg, params, prompt, steps=128, Tmax=256, rows=[0, 37])
    return cfg, params, prompt, toks, z, pos


def test_gpt2_bf16_decode_b64_prompt128_steps128(gpt2_decode_run):
    cfg, params, prompt, toks, z, pos = gpt2_decode_run
    assert pos == 256
    assert toks.shape == (64, 129)
    assert toks.min() >= 0 and toks.max() < cfg.vocab
    check_against_oracle(cfg, params, prompt, toks, z, [0, 37], bf16_tol, bf16_band)


def test_gpt2_bf16_decode_agrees_with_forward(gpt2_decode_run):
    # the cached path's logits at step s equal the full forward's logits at
    # position 127 + s of the same token sequence (both paths within 5e-2 of
    # the oracle, so within 1e-1 of each other), for all 64 sequences
    lib = _lib()
    cfg, params, prompt, toks, _, _ = gpt2_decode_run
    seq = np.concatenate([prompt, toks[:, :128]], axis=1)             # [64, 256]
    P = lib.params_to_device(cfg, synth.pack(cfg, params))
    dec = lib.Decoder(cfg, 64, 128, 256, poison=True)
    zstep = torch.empty((129, 64, cfg.vocab), dtype=torch.bfloat16, device="cuda")
    dec.prefill(P, torch.from_numpy(prompt).cuda(), last_logits=zstep[0])
    forced = torch.from_numpy(np.ascontiguousarray(toks[:, :128])).cuda()
    for s in range(128):
        dec.tok.copy_(forced[:, s])
        dec.step(P, logits=zstep[s + 1])
    f = lib.Forward(cfg, 64, 256, want_logits=True, poison=True)
    lg, _, _ = f(P, torch.from_numpy(seq).cuda())
    ref = lg[:, 127:256].float().permute(1, 0, 2)
    err = (zstep.float() - ref).abs().max().item()
    print(f"decode vs forward max|dlogit| {err:.4f}")
    assert err <= 1e-1


@pytest.mark.parametrize("n_embd,n_ff", [(64, 256), (64, 1536), (128, 1536)])
def test_decode_step_graph_replay_matches_eager(n_embd, n_ff):
    # one decode step captured in a HIP graph and replayed (the position is
    # read on the device), with eager work and synchronisations between
    # replays; every replay's tokens and logits equal the eager path's
    # (n_ff = 1536: split-K products, whose counters the step clears itself;
    # n_embd = 128: the step's products written as K-slices, reduced by the
    # attention and the residual LayerNorms)
    lib = _lib()
    cfg = synth.GPTConfig(vocab=257, ctx=64, n_embd=n_embd, n_head=2, n_layer=2, n_ff=n_ff, dtype=synth.BF16)
    params = synth.make_params(cfg, seed=6, cfg_id=9, init="stress")
    prompt = torch.from_numpy(synth.make_ids(cfg, 4, 10, seed=6, cfg_id=9)).cuda()
    P = lib.params_to_device(cfg, synth.pack(cfg, params))
    steps = 6

    eager = lib.Decoder(cfg, 4, 10, 32, poison=True)
    eager.prefill(P, prompt)
    ref_tok, ref_z = [], []
    for _ in range(steps):
        z = torch.empty((4, cfg.vocab), dtype=torch.bfloat16, device="cuda")
        eager.step(P, logits=z)
        ref_tok.append(eager.tok.clone())
        ref_z.append(z)
    torch.cuda.synchronize()

    g = lib.Decoder(cfg, 4, 10, 32, poison=True)
    zg = torch.empty((4, cfg.vocab), dtype=torch.bfloat16, device="cuda")
    g.prefill(P, prompt)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.step(P, logits=zg)
    for s in range(steps):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g.tok, ref_tok[s]), f"replay {s}: tokens differ"
        assert torch.equal(zg, ref_z[s]), f"replay {s}: logits differ"
        _ = (zg.float() * 2).sum().item()          # unrelated eager work between replays
    assert int(g.pos.item()) == 10 + steps
