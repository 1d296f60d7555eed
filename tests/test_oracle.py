"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the page passage it rests on.  The oracle is checked against
printed values (tests/golden), closed forms, identities, brute force, special
cases and CPU library routines (torch in float64 on the CPU, as an independent
cross-check only).  A mutation test at the end plants plausible mistakes in a
copy of the oracle and checks that these pins catch every one.
"""
import json
import math
import os

import numpy as np
import pytest

from decoder_only_transformer_attn_amd import synth
from oracle import gpt_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _model(cfg, seed=0, init="stress", **kw):
    p = synth.make_params(cfg, seed=seed, cfg_id=99, init=init, **kw)
    return synth.unpack_f64(cfg, p)


WALK = synth.GPTConfig(vocab=17, ctx=12, n_embd=8, n_head=2, n_layer=2, n_ff=32)
EX = synth.GPTConfig(vocab=11, ctx=10, n_embd=24, n_head=6, n_layer=1, n_ff=96)


# --------------------------------------------------------------------------
# Parameter count (第 25 章 §25.4; Day 16 三十一; 预训练一个 Mini GPT, KV cache)
# --------------------------------------------------------------------------
def test_param_count_printed_values():
    g = _gold("param_counts.json")
    t = g["gpt2_small_tied"]
    assert O.param_count(t["V"], t["C"], t["L"], t["ctx"]) == t["expected"]
    m = g["micro_tied"]
    assert O.param_count(m["V"], m["C"], m["L"], m["ctx"]) == m["expected"]
    u = g["gpt2_small_untied_extra"]
    assert u["V"] * u["C"] == u["expected"]
    # the MiniGPT tables are blob regions of exactly the printed sizes
    lay = {n: s for n, s, _ in synth.blob_layout(synth.MINI)[:-1]}
    assert int(np.prod(lay["wte"])) == g["minigpt_token_embedding"]["expected"]
    assert int(np.prod(lay["wpe"])) == g["minigpt_position_embedding"]["expected"]
    kv = g["kv_cache_values_per_token"]
    assert 2 * kv["L"] * kv["H"] * kv["D"] == kv["expected"]


@pytest.mark.parametrize("cfg", [synth.MICRO, synth.MINI, synth.GPT2, WALK, EX])
def test_blob_length_equals_closed_form(cfg):
    assert synth.blob_numel(cfg) == O.param_count(cfg.vocab, cfg.n_embd, cfg.n_layer, cfg.ctx, cfg.n_ff)


def test_param_count_sweep_matches_module_sum():
    # Day 16 三十六/三十七: sweep L and C; the closed form equals the sum of
    # the individual tensors' sizes, counted independently here.
    for L in (1, 2, 4, 8):
        for C in (64, 128, 256):
            V, ctx, F = 5000, 128, 4 * C
            attn = (3 * C * C + 3 * C) + (C * C + C)
            mlp = (F * C + F) + (C * F + C)
            lns = 2 * (2 * C)
            total = V * C + ctx * C + L * (attn + mlp + lns) + 2 * C
            assert O.param_count(V, C, L, ctx) == total


# --------------------------------------------------------------------------
# Shape walks (第 25 章 §25.2 and 练习; Day 16 四十一)
# --------------------------------------------------------------------------
def test_shape_walk_b2_t5_c8_h2():
    g = _gold("shape_walks.json")["walk"]
    params = _model(WALK)
    idx = synth.make_ids(WALK, g["B"], g["T"], seed=1)
    tr = {}
    logits, _, _ = O.forward(params, idx, WALK.n_head, trace=tr)
    assert list(tr["c_attn"]) == g["c_attn"]
    assert list(tr["split"]) == g["split"]
    assert list(tr["heads"]) == g["heads"]
    assert list(tr["scores"]) == g["scores"]
    assert logits.shape == (g["B"], g["T"], WALK.vocab)


def test_shape_walk_exercise_and_minigpt():
    g = _gold("shape_walks.json")
    e = g["exercise"]
    assert e["C"] // e["H"] == e["head_dim"]
    tr = {}
    O.forward(_model(EX), synth.make_ids(EX, e["B"], e["T"], seed=2), EX.n_head, trace=tr)
    assert list(tr["scores"]) == e["scores"]
    m = g["minigpt_debugger"]
    cfg = synth.GPTConfig(vocab=m["V"], ctx=128, n_embd=m["C"], n_head=m["H"], n_layer=1, n_ff=4 * m["C"])
    tr = {}
    logits, _, _ = O.forward(_model(cfg), synth.make_ids(cfg, m["B"], m["T"], seed=3), cfg.n_head, trace=tr)
    assert list(tr["heads"]) == m["heads"]
    assert list(tr["scores"]) == m["scores"]
    assert list(logits.shape) == m["logits"]


def test_sequence_too_long_and_bad_ids_raise():
    # Day 16 三十九: T > max_seq_len raises; ids live in [0, V) (§25.1)
    params = _model(synth.MICRO)
    with pytest.raises(ValueError):
        O.forward(params, np.zeros((1, 13), np.int32), 2)
    with pytest.raises(ValueError):
        O.forward(params, np.full((1, 4), 17, np.int32), 2)


# --------------------------------------------------------------------------
# LayerNorm (预训练一个 Mini GPT 第4步; GPT-1 notes §3.2)
# --------------------------------------------------------------------------
def test_layernorm_closed_form():
    rng = np.random.default_rng(0)
    for sigma in (1e-3, 0.1, 3.0):
        x = rng.standard_normal((7, 64)) * sigma + 5.0
        y = O.layer_norm(x, np.ones(64), np.zeros(64), 1e-5)
        var = x.var(axis=-1)  # biased
        np.testing.assert_allclose(y.mean(axis=-1), 0.0, atol=1e-12)
        np.testing.assert_allclose(y.var(axis=-1), var / (var + 1e-5), rtol=1e-10)
    # gain and bias act per channel
    g = rng.standard_normal(64)
    b = rng.standard_normal(64)
    base = O.layer_norm(x, np.ones(64), np.zeros(64))
    np.testing.assert_allclose(O.layer_norm(x, g, b), base * g + b, rtol=1e-12, atol=1e-12)


def test_layernorm_matches_torch_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 48)) * 2
    g, b = rng.standard_normal(48), rng.standard_normal(48)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (48,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(O.layer_norm(x, g, b, 1e-5), ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# GELU, tanh form (GPT-1 notes §3.6; 第 25 章 §25.3)
# --------------------------------------------------------------------------
def test_gelu_identities():
    x = np.linspace(-8, 8, 1001)
    np.testing.assert_allclose(O.gelu_tanh(x) - O.gelu_tanh(-x), x, atol=1e-13)
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    # large |x|: identity for x >> 0, zero for x << 0
    np.testing.assert_allclose(O.gelu_tanh(np.array([30.0, -30.0])), [30.0, 0.0], atol=1e-12)


def test_gelu_matches_torch_tanh_fp64_and_differs_from_erf():
    torch = pytest.importorskip("torch")
    x = np.linspace(-6, 6, 2001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(x), ref, rtol=1e-13, atol=1e-14)
    exact = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    assert np.abs(O.gelu_tanh(x) - exact).max() > 1e-4  # the tanh form is kept, not erf


# --------------------------------------------------------------------------
# Softmax (预训练一个 Mini GPT 第2步)
# --------------------------------------------------------------------------
def test_softmax_shift_invariance_and_normalisation():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((4, 9)) * 10
    p = O.softmax_rows(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14)
    np.testing.assert_allclose(O.softmax_rows(s - 123.0), p, atol=1e-15)
    big = O.softmax_rows(np.array([[1000.0, 1000.0, -np.inf]]))
    assert big[0, 2] == 0.0 and abs(big[0, 0] - 0.5) < 1e-15


# --------------------------------------------------------------------------
# Attention (第 25 章 §25.2; 预训练一个 Mini GPT 注意力)
# --------------------------------------------------------------------------
def test_attention_matches_brute_force():
    rng = np.random.default_rng(3)
    for T, D in ((1, 4), (5, 4), (7, 8), (12, 3)):
        q, k, u = (rng.standard_normal((T, D)) for _ in range(3))
        np.testing.assert_allclose(O.causal_attention(q, k, u), O.brute_attention(q, k, u),
                                   rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    rng = np.random.default_rng(4)
    T, D = 9, 8
    q, k, u = (rng.standard_normal((T, D)) for _ in range(3))
    y = O.causal_attention(q, k, u)
    np.testing.assert_array_equal(y[0], u[0])  # row 0 sees only itself
    y0 = O.causal_attention(np.zeros((T, D)), k, u)  # q = 0: uniform weights -> prefix mean
    prefix = np.cumsum(u, axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(y0, prefix, rtol=1e-13, atol=1e-14)


def test_attention_matches_torch_sdpa_causal_fp64():
    # 第 25 章 §25.2: the code calls scaled_dot_product_attention with is_causal=True;
    # this pins the 1/sqrt(D) scale and the s > t mask.
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    T, D = 11, 16
    q, k, u = (rng.standard_normal((T, D)) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(u)[None], is_causal=True)[0].numpy()
    np.testing.assert_allclose(O.causal_attention(q, k, u), ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# Linear orientation (第 25 章 §25.5)
# --------------------------------------------------------------------------
def test_linear_orientation_hand_worked():
    g = _gold("orientation.json")
    X, W, b, Y = (np.array(g[k], float) for k in ("X", "W", "b", "Y"))
    np.testing.assert_array_equal(O.linear(X, W, b), Y)
    Wsq = np.array([[1.0, 2.0], [3.0, 4.0]])  # asymmetric square: the two orientations differ
    assert not np.allclose(O.linear(X, Wsq), X @ Wsq)


# --------------------------------------------------------------------------
# Cross-entropy (预训练一个 Mini GPT 第6步; 第 25 章 §25.7)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [synth.MICRO, WALK])
def test_loss_is_log_v_when_embeddings_vanish(cfg):
    params = _model(cfg)
    params["wte"][:] = 0.0
    idx = synth.make_ids(cfg, 3, 6, seed=5)
    _, tok, mean = O.forward(params, idx, cfg.n_head)
    assert abs(mean - math.log(cfg.vocab)) < 1e-12
    np.testing.assert_allclose(tok[:, :-1], math.log(cfg.vocab), atol=1e-12)
    np.testing.assert_array_equal(tok[:, -1], 0.0)  # no target for the last position


def test_cross_entropy_matches_torch_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    z = rng.standard_normal((10, 37)) * 4
    y = rng.integers(0, 37, 10)
    y[3] = -1
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(z), torch.from_numpy(y),
                                            ignore_index=-1, reduction="none").numpy()
    np.testing.assert_allclose(O.cross_entropy_rows(z, y), ref, rtol=1e-13, atol=1e-13)


def test_derived_targets_shift_once():
    idx = np.array([[0, 1, 2, 3, 4]])
    np.testing.assert_array_equal(O.derived_targets(idx), [[1, 2, 3, 4, -1]])


def test_initial_loss_near_log_v():
    # 预训练一个 Mini GPT 第6步: a random model starts near ln(V)
    cfg = synth.MINI
    params = synth.unpack_f64(cfg, synth.make_params(cfg, seed=42, cfg_id=2))
    idx = synth.make_ids(cfg, 2, 32, seed=42, cfg_id=2)
    _, _, mean = O.forward(params, idx, cfg.n_head, want_logits=False)
    assert abs(mean - math.log(cfg.vocab)) < 0.1


# --------------------------------------------------------------------------
# Special cases of the whole model
# --------------------------------------------------------------------------
def _one_liner_l0(params, idx, eps=1e-5):
    x = params["wte"][idx] + params["wpe"][: idx.shape[1]]
    m = x.mean(-1, keepdims=True)
    v = ((x - m) ** 2).mean(-1, keepdims=True)
    return ((x - m) / np.sqrt(v + eps) * params["lnf_g"] + params["lnf_b"]) @ params["wte"].T


def test_zero_layers_is_embedding_then_tied_head():
    params = _model(synth.MICRO)
    params["layers"] = []
    idx = synth.make_ids(synth.MICRO, 2, 12, seed=7)
    logits, _, _ = O.forward(params, idx, 2)
    np.testing.assert_allclose(logits, _one_liner_l0(params, idx), rtol=1e-12, atol=1e-13)


def test_zeroed_residual_projections_make_blocks_identity():
    cfg = synth.MICRO
    p = synth.unpack_f64(cfg, synth.make_params(cfg, seed=8, cfg_id=9, init="stress", zero_residual_proj=True))
    idx = synth.make_ids(cfg, 2, 12, seed=8)
    logits, _, _ = O.forward(p, idx, cfg.n_head)
    np.testing.assert_allclose(logits, _one_liner_l0(p, idx), rtol=1e-12, atol=1e-13)


def test_tied_head_shares_the_token_table():
    # 第 25 章 §25.4: one tensor serves the lookup and the head
    cfg = synth.MICRO
    params = _model(cfg)
    idx = np.array([[1, 2, 3, 4]])
    base, _, _ = O.forward(params, idx, cfg.n_head)
    j = 9  # a token that is not in the input: only its logit column may change
    p2 = _model(cfg)
    p2["wte"][j] += 0.5
    pert, _, _ = O.forward(p2, idx, cfg.n_head)
    diff = np.abs(pert - base).max(axis=(0, 1))
    assert diff[j] > 1e-3 and np.all(np.delete(diff, j) == 0.0)
    # a token that is in the input at position 1: position 0 sees only the
    # changed logit column, later positions see a changed embedding too
    jj = int(idx[0, 1])
    p3 = _model(cfg)
    # not a constant shift: LayerNorm removes a shift common to all channels
    p3["wte"][jj] += np.linspace(-0.5, 0.5, cfg.n_embd)
    pert3, _, _ = O.forward(p3, idx, cfg.n_head)
    np.testing.assert_array_equal(np.delete(pert3[0, 0], jj), np.delete(base[0, 0], jj))
    assert abs(pert3[0, 0, jj] - base[0, 0, jj]) > 1e-3
    assert np.abs(np.delete(pert3[0, 1:], jj, axis=-1) - np.delete(base[0, 1:], jj, axis=-1)).max() > 1e-3


def test_causal_and_batch_invariance():
    cfg = synth.MICRO
    params = _model(cfg)
    idx = synth.make_ids(cfg, 3, 12, seed=9)
    base, _, _ = O.forward(params, idx, cfg.n_head)
    for t in (0, 5, 10):
        idx2 = idx.copy()
        idx2[1, t + 1:] = (idx2[1, t + 1:] + 3) % cfg.vocab
        pert, _, _ = O.forward(params, idx2, cfg.n_head)
        np.testing.assert_array_equal(pert[1, : t + 1], base[1, : t + 1])
        assert np.abs(pert[1, t + 1:] - base[1, t + 1:]).max() > 0
        np.testing.assert_array_equal(pert[[0, 2]], base[[0, 2]])


def test_model_matches_torch_functional_fp64():
    # Independent composition from CPU library routines (layer_norm, linear,
    # gelu tanh, SDPA causal, cross_entropy) in float64.
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    cfg = synth.MICRO
    params = _model(cfg, seed=10)
    idx = synth.make_ids(cfg, 3, 12, seed=10)
    t = {k: torch.from_numpy(v) for k, v in params.items() if isinstance(v, np.ndarray)}
    x = t["wte"][torch.from_numpy(idx.astype(np.int64))] + t["wpe"][:12]
    H, C = cfg.n_head, cfg.n_embd
    for lp in params["layers"]:
        lp = {k: torch.from_numpy(v) for k, v in lp.items()}
        a = F.layer_norm(x, (C,), lp["ln1_g"], lp["ln1_b"], 1e-5)
        q, k, v = F.linear(a, lp["attn_w"], lp["attn_b"]).split(C, dim=-1)
        sh = lambda z: z.view(3, 12, H, C // H).transpose(1, 2)
        y = F.scaled_dot_product_attention(sh(q), sh(k), sh(v), is_causal=True)
        x = x + F.linear(y.transpose(1, 2).reshape(3, 12, C), lp["proj_w"], lp["proj_b"])
        a = F.layer_norm(x, (C,), lp["ln2_g"], lp["ln2_b"], 1e-5)
        x = x + F.linear(F.gelu(F.linear(a, lp["fc_w"], lp["fc_b"]), approximate="tanh"),
                         lp["fcproj_w"], lp["fcproj_b"])
    z = F.layer_norm(x, (C,), t["lnf_g"], t["lnf_b"], 1e-5) @ t["wte"].T
    ref_loss = F.cross_entropy(z[:, :-1].reshape(-1, cfg.vocab),
                               torch.from_numpy(idx[:, 1:].astype(np.int64)).reshape(-1))
    logits, _, mean = O.forward(params, idx, cfg.n_head)
    np.testing.assert_allclose(logits, z.numpy(), rtol=1e-11, atol=1e-12)
    assert abs(mean - float(ref_loss)) < 1e-12


# --------------------------------------------------------------------------
# KV cache (预训练一个 Mini GPT, KV cache; GPT-1 notes §6.1 greedy)
# --------------------------------------------------------------------------
def test_kv_cache_decode_equals_recompute():
    cfg = synth.MICRO
    params = _model(cfg, seed=11)
    prompt = synth.make_ids(cfg, 3, 5, seed=11)
    t1, z1 = O.greedy_recompute(params, prompt, 6, cfg.n_head)
    t2, z2 = O.greedy_cached(params, prompt, 6, cfg.n_head)
    np.testing.assert_array_equal(t1, t2)
    np.testing.assert_allclose(z1, z2, rtol=1e-12, atol=1e-12)
    # step logits equal the full forward's logits at the same positions
    seq = np.concatenate([prompt, t1[:, :-1]], axis=1)
    full, _, _ = O.forward(params, seq, cfg.n_head)
    np.testing.assert_allclose(z2, full[:, prompt.shape[1] - 1:], rtol=1e-12, atol=1e-12)


def test_argmax_lowest_index_on_ties():
    assert O.argmax_lowest(np.array([[1.0, 3.0, 3.0, 2.0]]))[0] == 1


# --------------------------------------------------------------------------
# Mutation check: plausible mistakes planted in the oracle (on the CPU) must
# each fail at least one of the pins above.
# --------------------------------------------------------------------------
def _pins_pass():
    checks = [test_layernorm_closed_form, test_gelu_identities, test_attention_closed_forms,
              test_linear_orientation_hand_worked, test_zero_layers_is_embedding_then_tied_head,
              test_causal_and_batch_invariance, test_kv_cache_decode_equals_recompute,
              lambda: test_loss_is_log_v_when_embeddings_vanish(synth.MICRO)]
    torch_checks = [test_layernorm_matches_torch_fp64, test_gelu_matches_torch_tanh_fp64_and_differs_from_erf,
                    test_attention_matches_torch_sdpa_causal_fp64, test_model_matches_torch_functional_fp64,
                    test_cross_entropy_matches_torch_fp64]
    for c in checks + torch_checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


def test_pins_catch_planted_mistakes(monkeypatch):
    assert _pins_pass()
    sq = math.sqrt

    def ln_unbiased(x, g, b, eps=1e-5):
        m = x.mean(-1, keepdims=True)
        return g * (x - m) / np.sqrt(x.var(-1, ddof=1, keepdims=True) + eps) + b

    def ln_eps_outside(x, g, b, eps=1e-5):
        m = x.mean(-1, keepdims=True)
        return g * (x - m) / (np.sqrt(x.var(-1, keepdims=True)) + eps) + b

    def gelu_wrong_const(z):
        return 0.5 * z * (1.0 + np.tanh(sq(2.0 / math.pi) * (z + 0.0447 * z ** 3)))

    def attn_wrong_scale(q, k, u):
        T, D = q.shape
        s = (q @ k.T) / D
        s = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, s)
        return O.softmax_rows(s) @ u

    def attn_mask_off_by_one(q, k, u):
        T, D = q.shape
        s = (q @ k.T) / sq(D)
        s = np.where(np.triu(np.ones((T, T), bool), 2), -np.inf, s)
        return O.softmax_rows(s) @ u

    def linear_transposed(x, W, b=None):
        # square weights silently used in the other orientation
        y = x @ W if W.shape[0] == W.shape[1] else x @ W.T
        return y if b is None else y + b

    def ce_mean_not_sum(z, y):
        lse = np.log(np.exp(z).mean(-1))
        yy = np.where(y >= 0, y, 0)
        return np.where(y >= 0, lse - z[np.arange(len(y)), yy], 0.0)

    def targets_shifted_twice(idx):
        idx = np.asarray(idx)
        y = np.full(idx.shape, -1, dtype=np.int64)
        y[:, :-2] = idx[:, 2:]
        return y

    def head_untied(params, a):
        return a @ (params["wte"][::-1]).T

    mutants = [("layer_norm", ln_unbiased), ("layer_norm", ln_eps_outside), ("gelu_tanh", gelu_wrong_const),
               ("causal_attention", attn_wrong_scale), ("causal_attention", attn_mask_off_by_one),
               ("linear", linear_transposed), ("cross_entropy_rows", ce_mean_not_sum), ("head", head_untied),
               ("derived_targets", targets_shifted_twice)]
    for name, fn in mutants:
        with monkeypatch.context() as m:
            m.setattr(O, name, fn)
            assert not _pins_pass(), f"planted mistake in {name} ({fn.__name__}) went unnoticed"
