"""GPU parity of the sampler (gpt_sample through the C ABI) against the
float64 sampling oracle on the same logits, seen sets and uniforms.

The oracle decides in float64 (the precision of the Mini-GPT lesson's numpy
sampler, 构建它 第7步); the kernel forms the penalised key in float32 and
rounds each weight exp(key - max) to float32 before summing in double.  A
GPU token is accepted when it equals the oracle's draw, or when it is a
correct draw under the float64 distribution up to that rounding
(``valid_draw``): it survives top-k and top-p under some order of the
candidates whose keys lie within the rounding bound tau of each other, and
u * Z lies inside its cumulative-mass interval widened by 2 tau Z.  The
bound follows from the kernel's arithmetic: two float32 divisions give
|key_f32 - key| <= 2^-23 |key|, so every weight and mass is within
tau = 2^-22 (2 max|key| + 1) (relative; a factor 2 of margin) of the float64
value.  Every test also reports how many tokens differ from the oracle's
own draw.  Logit rows cover flat and peaked distributions, many ties
(integer logits), ragged vocabularies and the full GPT-2 vocabulary;
settings cover greedy, plain temperature, top-k, top-p, their combination
and the repetition penalty ("02 GPT 架构" 第 8 章 §8.1-§8.4).
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


def _tau(key):
    return 2.0 ** -22 * (2.0 * float(np.abs(key).max()) + 1.0)


def valid_draw(z, seen, t, k, p, a, u, tok):
    """True when tok is a correct draw from the float64 filtered distribution
    of the row z, up to the kernel's float32 rounding of keys and weights."""
    V = z.size
    if not 0 <= tok < V:
        return False
    if t <= 0:   # greedy on the penalised logits
        key = S.penalize(z, seen, a)
        return key[tok] >= key.max() - _tau(key)
    key = S.keys(z, seen, t, a)
    tau = _tau(key)
    w = np.exp(key - key.max())
    order = S.candidate_order(w)
    kk = k if 0 < k < V else V
    topk = order[:kk]
    # before tok in every admissible order: keys larger beyond the bound, and
    # exact ties at lower indices (equal float64 keys are equal in float32,
    # and both sides break such ties by index)
    idx = np.arange(V)
    heavier = (key > key[tok] + tau) | ((key == key[tok]) & (idx < tok))
    near = (np.abs(key - key[tok]) <= tau) & (key != key[tok])   # may fall either side of tok
    if heavier.sum() >= kk:                           # tok cannot be among the k largest
        return False
    in_k = np.zeros(V, bool)
    in_k[topk] = True
    # near ties straddling the k-th place can each be kept
    if 0 < k < V:
        in_k |= (np.abs(key - key[topk[-1]]) <= tau) & (key != key[topk[-1]])
    Zk = float(w[topk].sum())
    cum = np.cumsum(w[topk])
    # nucleus sizes consistent with the rounding (the oracle's, or one either
    # side when p Zk lies within 2 tau Zk of a cumulative boundary)
    sizes = [len(topk)]
    if p < 1.0:
        X = p * Zk
        n0 = int(np.searchsorted(cum, X, side="left")) + 1
        sizes = [n for n in (n0 - 1, n0, n0 + 1)
                 if 1 <= n <= len(topk) and cum[n - 1] >= X - 2 * tau * Zk
                 and (n == 1 or cum[n - 2] < X + 2 * tau * Zk)]
    lo = float(w[heavier & in_k].sum())
    hi = lo + float(w[near & in_k].sum()) + float(w[tok])
    for n in sizes:
        if (heavier & in_k).sum() >= n:               # tok cannot be among the first n
            continue
        r = float(u) * float(cum[n - 1])
        if lo - 2 * tau * Zk <= r <= hi + 2 * tau * Zk:
            return True
    return False


def check_rows(zin, seen, t, k, p, a, u, got, what):
    """Every GPU token valid; returns the number that differ from the oracle's draw."""
    ref = S.sample_rows(zin, seen, t, k, p, a, u)
    bad = [b for b in range(zin.shape[0])
           if got[b] != ref[b] and not valid_draw(zin[b], None if seen is None else seen[b], t, k, p, a, u[b],
                                                  int(got[b]))]
    assert not bad, f"{what}: invalid draws in rows {bad[:8]} (gpu {got[bad[:8]]}, oracle {ref[bad[:8]]})"
    return int((got != ref).sum())


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
        g = got.cpu().numpy()
        diff = check_rows(zin, seen0, t, k, p, a, u, g, f"settings {(t, k, p, a)}")
        if diff:
            print(f"V={V} B={B} {kind} {(t, k, p, a)}: {diff} of {B} tokens differ from the oracle's draw (valid)")
        # the chosen tokens' bits are set, the others unchanged
        after = _unbits(seen.cpu().numpy(), V)
        expect = seen0.copy()
        expect[np.arange(B), g] = True
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
    check_rows(zt.float().cpu().numpy(), None, 0.9, 0, 0.92, 1.2, u.cpu().numpy(), a, "no seen set")


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
    # the case is well posed: p Z lies far from every cumulative boundary of
    # the top-k set, so the float32 rounding cannot change the nucleus
    ck, wk = S.filtered(z, None, 0.9, 10, 1.0)
    assert np.min(np.abs(np.cumsum(wk) - 0.8 * wk.sum())) > 1e-4 * wk.sum()
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
    dec = lib.Decoder(cfg, B, Tp, 32, poison=True)
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
        g = tok.cpu().numpy()
        check_rows(z.float().cpu().numpy(), seen, 0.9, 40, 0.9, 1.2, u, g, f"emission {it}")
        seen[np.arange(B), g] = True
    assert int(dec.pos.item()) == Tp + steps
