"""Pins of the backward oracle (oracle/grad_oracle.py).

* central finite differences of the forward oracle's mean loss (an
  independent computation: only gpt_oracle.forward is evaluated), for every
  parameter of models without blocks (tied, untied, pre- and post-LN) and for
  the rows entering the final LayerNorm;
* torch float64 autograd of the same composition (library routines);
* invariants: each row of dz sums to zero and rows without a target are zero,
  so the head gradient's columns sum to zero; LayerNorm input gradients sum to
  zero over each row (the output ignores a shift of the row);
* planted mistakes, each of which one of the above must catch.
"""
import dataclasses as dc

import numpy as np
import pytest

from decoder_only_transformer_attn_amd import synth
from oracle import gpt_oracle as O
from oracle import grad_oracle as G

BASE = synth.GPTConfig(vocab=19, ctx=12, n_embd=16, n_head=2, n_layer=0, n_ff=64)


def _P(cfg, seed=0):
    return synth.unpack_f64(cfg, synth.make_params(cfg, seed=seed, cfg_id=91, init="stress"))


def _loss(P, idx, targets=None):
    return O.forward(P, idx, BASE.n_head, targets=targets, want_logits=False)[2]


def _fd(P, idx, key, entries, targets=None, h=1e-5):
    out = []
    for e in entries:
        arr = P[key]
        old = arr[e]
        arr[e] = old + h
        lp = _loss(P, idx, targets)
        arr[e] = old - h
        lm = _loss(P, idx, targets)
        arr[e] = old
        out.append((lp - lm) / (2 * h))
    return np.array(out)


def _entries(shape, rng, n=12, rows=None):
    r = rng.integers(0, shape[0], n) if rows is None else np.asarray(rows)
    return [(int(a), int(b)) if len(shape) == 2 else (int(a),) for a, b in
            zip(r, rng.integers(0, shape[-1], len(r)))]


@pytest.mark.parametrize("post_ln,untied", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_no_block_gradients_match_finite_differences(post_ln, untied):
    cfg = dc.replace(BASE, post_ln=post_ln, untied=untied)
    P = _P(cfg, seed=post_ln + 2 * untied)
    rng = np.random.default_rng(5)
    idx = synth.make_ids(cfg, 3, 9, seed=5)
    g = G.grads_no_blocks(P, idx)
    assert abs(g["loss"] - _loss(P, idx)) < 1e-12
    # token-table rows that appear in the input (both uses) and rows that do not (head only)
    present = np.unique(idx)
    absent = np.setdiff1d(np.arange(cfg.vocab), present)
    rows = np.concatenate([present[:6], absent[:4]])
    checks = [("wte", _entries(P["wte"].shape, rng, rows=rows)), ("wpe", _entries(P["wpe"].shape, rng))]
    if not post_ln:
        checks += [("lnf_g", _entries(P["lnf_g"].shape, rng, n=6)), ("lnf_b", _entries(P["lnf_b"].shape, rng, n=6))]
    if untied:
        checks.append(("head_w", _entries(P["head_w"].shape, rng)))
    for key, ent in checks:
        fd = _fd(P, idx, key, ent)
        an = np.array([g[key][e] for e in ent])
        np.testing.assert_allclose(an, fd, rtol=1e-6, atol=1e-9, err_msg=key)
    # positions past T get no gradient
    assert np.all(g["wpe"][9:] == 0)


def test_explicit_targets_with_ignored_positions():
    P = _P(BASE, seed=3)
    idx = synth.make_ids(BASE, 2, 7, seed=6)
    tg = np.random.default_rng(6).integers(0, BASE.vocab, (2, 7))
    tg[0, 2] = tg[1, 5] = tg[1, 6] = -1
    g = G.grads_no_blocks(P, idx, tg)
    rng = np.random.default_rng(7)
    for key in ("wte", "wpe", "lnf_g"):
        ent = _entries(P[key].shape, rng, n=8)
        np.testing.assert_allclose([g[key][e] for e in ent], _fd(P, idx, key, ent, tg), rtol=1e-6, atol=1e-9)


def test_head_backward_dx_matches_finite_differences():
    # loss as a function of the rows entering the final LayerNorm
    P = _P(BASE, seed=8)
    rng = np.random.default_rng(8)
    N, C = 10, BASE.n_embd
    x = rng.normal(0, 2, (N, C))
    y = rng.integers(0, BASE.vocab, N)
    y[3] = -1
    hb = G.head_backward(P, x, y)

    def loss(xx):
        z = O.head(P, O.layer_norm(xx, P["lnf_g"], P["lnf_b"]))
        v = y >= 0
        return O.cross_entropy_rows(z, y)[v].sum() / v.sum()

    assert abs(hb["loss"] - loss(x)) < 1e-12
    h = 1e-5
    for (i, j) in _entries((N, C), rng, n=16):
        xp, xm = x.copy(), x.copy()
        xp[i, j] += h
        xm[i, j] -= h
        assert abs(hb["dx"][i, j] - (loss(xp) - loss(xm)) / (2 * h)) < 1e-8
    np.testing.assert_allclose(hb["dx"][3], 0.0, atol=0)   # no target: no gradient through its row


def test_matches_torch_autograd_fp64():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    cfg = dc.replace(BASE, vocab=37, n_embd=24, n_head=3)
    P = _P(cfg, seed=9)
    idx = synth.make_ids(cfg, 2, 11, seed=9)
    g = G.grads_no_blocks(P, idx)
    wte = torch.tensor(P["wte"], requires_grad=True)
    wpe = torch.tensor(P["wpe"], requires_grad=True)
    lg = torch.tensor(P["lnf_g"], requires_grad=True)
    lb = torch.tensor(P["lnf_b"], requires_grad=True)
    it = torch.from_numpy(idx)
    x = F.embedding(it, wte) + wpe[: idx.shape[1]]
    z = F.linear(F.layer_norm(x, (cfg.n_embd,), lg, lb, 1e-5), wte)
    y = torch.from_numpy(O.derived_targets(idx))
    loss = F.cross_entropy(z.reshape(-1, cfg.vocab), y.reshape(-1), ignore_index=-1)
    loss.backward()
    assert abs(loss.item() - g["loss"]) < 1e-12
    for name, t in (("wte", wte), ("wpe", wpe), ("lnf_g", lg), ("lnf_b", lb)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-13, err_msg=name)


def test_invariants():
    P = _P(BASE, seed=10)
    rng = np.random.default_rng(10)
    a = rng.normal(0, 1, (9, BASE.n_embd))
    y = rng.integers(0, BASE.vocab, 9)
    y[[1, 4]] = -1
    dz, da, dW, _ = G.ce_head_backward(P, a, y)
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-15)
    assert np.all(dz[[1, 4]] == 0)
    np.testing.assert_allclose(dW.sum(axis=0), 0.0, atol=1e-14)
    # each valid row: the target entry is the only negative one, p - 1 over n_valid
    for n in np.nonzero(y >= 0)[0]:
        assert dz[n, y[n]] < 0 and np.all(np.delete(dz[n], y[n]) > 0)
    x = rng.normal(0, 3, (9, BASE.n_embd))
    dx, _, _ = G.layer_norm_backward(x, P["lnf_g"], rng.normal(0, 1, (9, BASE.n_embd)))
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-13)


def test_embedding_backward_brute_force():
    rng = np.random.default_rng(11)
    idx = np.array([[3, 1, 3, 0], [1, 1, 2, 3]])
    dx0 = rng.normal(0, 1, (2, 4, 5))
    dE, dP = G.embedding_backward(idx, dx0, 6, 7)
    np.testing.assert_allclose(dE[3], dx0[0, 0] + dx0[0, 2] + dx0[1, 3])
    np.testing.assert_allclose(dE[1], dx0[0, 1] + dx0[1, 0] + dx0[1, 1])
    assert np.all(dE[4] == 0) and np.all(dE[5] == 0)
    np.testing.assert_allclose(dP[:4], dx0[0] + dx0[1])
    assert np.all(dP[4:] == 0)


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------
def _pins_pass():
    try:
        test_no_block_gradients_match_finite_differences(0, 0)
        test_head_backward_dx_matches_finite_differences()
        test_invariants()
    except AssertionError:
        return False
    return True


def test_pins_catch_planted_mistakes(monkeypatch):
    assert _pins_pass()
    orig_ce, orig_ln, orig_emb = G.ce_head_backward, G.layer_norm_backward, G.embedding_backward

    def ce_without_mean(params, a, y):
        dz, da, dW, loss = orig_ce(params, a, y)
        n = int((np.asarray(y) >= 0).sum())
        return dz * n, da * n, dW * n, loss

    def ce_softmax_only(params, a, y):
        W = params.get("head_w", params["wte"])
        y = np.asarray(y)
        dz = O.softmax_rows(a @ W.T) / max(1, int((y >= 0).sum()))
        dz[y < 0] = 0
        return dz, dz @ W, dz.T @ a, 0.0

    def ln_missing_term(x, g, dy, eps=1e-5):
        mu = x.mean(axis=-1, keepdims=True)
        r = 1.0 / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
        gd = dy * g
        dx = r * (gd - gd.mean(axis=-1, keepdims=True))
        _, dg, db = orig_ln(x, g, dy, eps)
        return dx, dg, db

    def embedding_head_share_only(idx, dx0, vocab, ctx):
        _, dP = orig_emb(idx, dx0, vocab, ctx)
        return np.zeros((vocab, dx0.shape[-1])), dP

    mutants = [("ce_head_backward", ce_without_mean), ("ce_head_backward", ce_softmax_only),
               ("layer_norm_backward", ln_missing_term), ("embedding_backward", embedding_head_share_only)]
    for name, fn in mutants:
        with monkeypatch.context() as m:
            m.setattr(G, name, fn)
            assert not _pins_pass(), f"planted mistake {fn.__name__} went unnoticed"


# --------------------------------------------------------------------------
# block backward and the full model
# --------------------------------------------------------------------------
BLK = synth.GPTConfig(vocab=23, ctx=12, n_embd=16, n_head=2, n_layer=2, n_ff=48)


def _block_f(x, lp, dy, act="tanh"):
    return float((dy * O.block(x, lp, BLK.n_head, 1e-5, act=act)).sum())


@pytest.mark.parametrize("act", ["tanh", "erf"])
def test_block_backward_matches_finite_differences(act):
    P = _P(dc.replace(BLK, act=1 if act == "erf" else 0), seed=12)
    lp = P["layers"][0]
    rng = np.random.default_rng(12)
    x = rng.normal(0, 1.5, (2, 7, BLK.n_embd))
    dy = rng.normal(0, 1, x.shape)
    dx, g = G.block_backward(x, lp, dy, BLK.n_head, 1e-5, act)
    h = 1e-5
    for idx in [(0, 0, 0), (1, 6, 15), (0, 3, 7), (1, 2, 9)]:
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd = (_block_f(xp, lp, dy, act) - _block_f(xm, lp, dy, act)) / (2 * h)
        assert abs(dx[idx] - fd) < 1e-7 * max(1.0, abs(fd)), ("x", idx)
    for key, arr in lp.items():
        for e in _entries(arr.shape, rng, n=3):
            old = arr[e]
            arr[e] = old + h
            fp = _block_f(x, lp, dy, act)
            arr[e] = old - h
            fm = _block_f(x, lp, dy, act)
            arr[e] = old
            fd = (fp - fm) / (2 * h)
            assert abs(g[key][e] - fd) < 1e-7 * max(1.0, abs(fd)), (key, e, g[key][e], fd)


def test_attention_backward_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    q, k, u, dy = (rng.normal(size=(9, 8)) for _ in range(4))
    tq, tk, tu = (torch.tensor(a, requires_grad=True) for a in (q, k, u))
    y = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tu[None], is_causal=True)[0]
    y.backward(torch.from_numpy(dy))
    for got, t in zip(G.attention_backward(q, k, u, dy), (tq, tk, tu)):
        np.testing.assert_allclose(got, t.grad.numpy(), atol=1e-13)


def test_gelu_grads_match_torch():
    torch = pytest.importorskip("torch")
    z = torch.linspace(-6, 6, 241, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(z, approximate="tanh").sum().backward()
    np.testing.assert_allclose(G.gelu_tanh_grad(z.detach().numpy()), z.grad.numpy(), atol=1e-14)
    z.grad = None
    torch.nn.functional.gelu(z).sum().backward()
    np.testing.assert_allclose(G.gelu_erf_grad(z.detach().numpy()), z.grad.numpy(), atol=1e-14)


def test_full_gradients_match_finite_differences():
    P = _P(BLK, seed=14)
    idx = synth.make_ids(BLK, 2, 8, seed=14)
    g = G.grads_full(P, idx, BLK.n_head)
    assert abs(g["loss"] - _loss(P, idx)) < 1e-12
    rng = np.random.default_rng(14)
    h = 1e-5
    for key in ("wte", "wpe", "lnf_g", "lnf_b"):
        ent = _entries(P[key].shape, rng, n=4)
        np.testing.assert_allclose([g[key][e] for e in ent], _fd(P, idx, key, ent), rtol=1e-6, atol=1e-9,
                                   err_msg=key)
    for l in range(BLK.n_layer):
        lp = P["layers"][l]
        for key, arr in lp.items():
            for e in _entries(arr.shape, rng, n=2):
                old = arr[e]
                arr[e] = old + h
                lp_ = _loss(P, idx)
                arr[e] = old - h
                lm = _loss(P, idx)
                arr[e] = old
                fd = (lp_ - lm) / (2 * h)
                assert abs(g["layers"][l][key][e] - fd) < 1e-6 * max(1e-3, abs(fd)) + 1e-9, (l, key, e)


def test_full_gradients_match_torch_autograd():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    P = _P(BLK, seed=15)
    idx = synth.make_ids(BLK, 2, 9, seed=15)
    g = G.grads_full(P, idx, BLK.n_head)
    T = {k: torch.tensor(v, requires_grad=True) for k, v in P.items() if isinstance(v, np.ndarray)}
    L = [{k: torch.tensor(v, requires_grad=True) for k, v in lp.items()} for lp in P["layers"]]
    B, Tn, C, H = 2, 9, BLK.n_embd, BLK.n_head
    x = F.embedding(torch.from_numpy(idx), T["wte"]) + T["wpe"][:Tn]
    for lp in L:
        a = F.layer_norm(x, (C,), lp["ln1_g"], lp["ln1_b"], 1e-5)
        q, k, v = F.linear(a, lp["attn_w"], lp["attn_b"]).split(C, dim=-1)
        sh = lambda z: z.view(B, Tn, H, C // H).transpose(1, 2)
        y = F.scaled_dot_product_attention(sh(q), sh(k), sh(v), is_causal=True).transpose(1, 2).reshape(B, Tn, C)
        x = x + F.linear(y, lp["proj_w"], lp["proj_b"])
        a = F.layer_norm(x, (C,), lp["ln2_g"], lp["ln2_b"], 1e-5)
        x = x + F.linear(F.gelu(F.linear(a, lp["fc_w"], lp["fc_b"]), approximate="tanh"), lp["fcproj_w"],
                         lp["fcproj_b"])
    z = F.linear(F.layer_norm(x, (C,), T["lnf_g"], T["lnf_b"], 1e-5), T["wte"])
    F.cross_entropy(z.reshape(-1, BLK.vocab), torch.from_numpy(O.derived_targets(idx)).reshape(-1),
                    ignore_index=-1).backward()
    for key in ("wte", "wpe", "lnf_g", "lnf_b"):
        np.testing.assert_allclose(g[key], T[key].grad.numpy(), rtol=1e-9, atol=1e-12, err_msg=key)
    for l in range(BLK.n_layer):
        for key, t in L[l].items():
            np.testing.assert_allclose(g["layers"][l][key], t.grad.numpy(), rtol=1e-9, atol=1e-12,
                                       err_msg=f"{l}.{key}")


def _block_pins_pass():
    try:
        test_block_backward_matches_finite_differences("tanh")
        test_attention_backward_matches_torch()
        test_gelu_grads_match_torch()
    except AssertionError:
        return False
    return True


def test_block_pins_catch_planted_mistakes(monkeypatch):
    pytest.importorskip("torch")
    assert _block_pins_pass()
    orig_attn, orig_blk = G.attention_backward, G.block_backward

    def attn_without_rowsum(q, k, u, dy):
        T, D = q.shape
        s = np.where(np.triu(np.ones((T, T), dtype=bool), k=1), -np.inf, (q @ k.T) / np.sqrt(D))
        p = O.softmax_rows(s)
        ds = p * (dy @ u.T)
        return ds @ k / np.sqrt(D), ds.T @ q / np.sqrt(D), p.T @ dy

    def gelu_grad_one(z):
        return np.ones_like(z)

    def blk_dropping_residual(x, lp, dy, n_head, eps=1e-5, act="tanh"):
        dx, g = orig_blk(x, lp, dy, n_head, eps, act)
        return dx - dy, g

    def blk_bias_sign_flipped(x, lp, dy, n_head, eps=1e-5, act="tanh"):
        dx, g = orig_blk(x, lp, dy, n_head, eps, act)
        g = dict(g)
        g["fcproj_b"] = -g["fcproj_b"]
        return dx, g

    for name, fn in [("attention_backward", attn_without_rowsum), ("gelu_tanh_grad", gelu_grad_one),
                     ("block_backward", blk_dropping_residual), ("block_backward", blk_bias_sign_flipped)]:
        with monkeypatch.context() as m:
            m.setattr(G, name, fn)
            assert not _block_pins_pass(), f"planted mistake {fn.__name__} went unnoticed"
