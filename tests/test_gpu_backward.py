"""GPU parity of the loss backward through the head, the final LayerNorm and
the embeddings (gpt_head_backward, gpt_embedding_backward through the C ABI)
against the fp64 backward oracle on the same inputs.

Tolerances (max |GPU - oracle| over max |oracle|, per output):
  fp32: 1e-4 (fp32 products and accumulation, exp2 / log of the loss
        kernels: relative errors of a few 1e-6);
  bf16: 3e-2 for dx and the head gradient (the final hidden rows and dz are
        rounded to bf16, 2^-9 relative each, and the logits they produce
        differ from the oracle's fp64 ones by about 2^-9 |z|; the softmax
        turns that into about 1% of each probability), 1e-2 for the
        LayerNorm gain/bias sums and the loss.
The embedding backward adds fp32 rows in position order: 1e-5 relative.
"""
import dataclasses as dc

import numpy as np
import pytest

from decoder_only_transformer_attn_amd import synth
from oracle import gpt_oracle as O
from oracle import grad_oracle as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = {synth.F32: dict(g=1e-4, s=1e-4), synth.BF16: dict(g=3e-2, s=1e-2)}


def _lib():
    from decoder_only_transformer_attn_amd import lib
    lib.load()
    return lib


def _rel(got, ref):
    return float(np.abs(np.asarray(got, np.float64) - ref).max() / max(np.abs(ref).max(), 1e-30))


def _slot(lib, cfg, name):
    """(offset, shape) of a named tensor in the parameter / gradient blob."""
    for nm, shape, off in synth.blob_layout(cfg):
        if nm == name:
            return off, shape
    raise KeyError(name)


def _run_head_backward(lib, cfg, params, idx, x, targets=None, g0_scale=1e-3, seed=0):
    P = lib.params_to_device(cfg, synth.pack(cfg, params))
    B, T = idx.shape
    n = lib.param_count(cfg)
    g0 = (np.random.default_rng(seed).normal(0, g0_scale, n)).astype(np.float32)
    grads = torch.from_numpy(g0).cuda()
    xd = torch.from_numpy(x.astype(np.float32)).cuda()
    dx = torch.full_like(xd, float("nan"))
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.head_backward_workspace_bytes(cfg, B, T), dtype=torch.uint8, device="cuda")
    tg = None if targets is None else torch.from_numpy(targets.astype(np.int32)).cuda()
    lib.head_backward(cfg, P, torch.from_numpy(idx.astype(np.int32)).cuda(), xd, dx, grads, tg, loss, ws)
    torch.cuda.synchronize()
    return dx.cpu().numpy(), grads.cpu().numpy().astype(np.float64) - g0, float(loss.item())


def _head_name(cfg):
    return "head_w" if cfg.untied else "wte"


CASES = [  # vocab, C, L, B, T, post_ln, untied
    (1000, 64, 1, 3, 37, 0, 0),
    (1000, 64, 1, 2, 9, 0, 0),      # at most 64 rows
    (517, 128, 2, 2, 40, 1, 0),     # post-LN: the head reads x itself
    (517, 128, 1, 2, 40, 0, 1),     # untied head matrix
    (333, 64, 0, 4, 21, 1, 1),
]


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("case", CASES)
def test_head_backward_matches_oracle(dtype, case):
    lib = _lib()
    V, C, L, B, T, post, untied = case
    cfg = synth.GPTConfig(vocab=V, ctx=64, n_embd=C, n_head=2, n_layer=L, n_ff=2 * C, dtype=dtype, post_ln=post,
                          untied=untied)
    params = synth.make_params(cfg, seed=V + C, cfg_id=31, init="stress")
    Pf = synth.unpack_f64(cfg, params)
    rng = np.random.default_rng(V * 7 + T)
    idx = synth.make_ids(cfg, B, T, seed=V + T)
    x = rng.normal(0, 1.5, (B * T, C)).astype(np.float32)
    targets = O.derived_targets(idx)
    targets[0, 3] = -1
    dx, dg, loss = _run_head_backward(lib, cfg, params, idx, x, targets)
    ref = G.head_backward(Pf, x.astype(np.float64), targets.reshape(-1))
    tol = TOL[dtype]
    assert np.isfinite(dx).all()
    assert _rel(dx, ref["dx"]) <= tol["g"], ("dx", _rel(dx, ref["dx"]))
    off, shape = _slot(lib, cfg, _head_name(cfg))
    got_w = dg[off:off + V * C].reshape(V, C)
    assert _rel(got_w, ref["head"]) <= tol["g"], ("head", _rel(got_w, ref["head"]))
    if not post:
        for nm in ("lnf_g", "lnf_b"):
            o, _ = _slot(lib, cfg, nm)
            assert _rel(dg[o:o + C], ref[nm]) <= tol["s"], (nm, _rel(dg[o:o + C], ref[nm]))
    assert abs(loss - ref["loss"]) <= tol["s"] * abs(ref["loss"])
    # nothing else in the gradient blob changed
    touched = np.zeros(dg.shape, bool)
    touched[off:off + V * C] = True
    if not post:
        for nm in ("lnf_g", "lnf_b"):
            o, _ = _slot(lib, cfg, nm)
            touched[o:o + C] = True
    assert np.all(dg[~touched] == 0)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("post_ln,untied", [(0, 0), (1, 0), (0, 1)])
def test_full_gradient_of_a_model_without_blocks(dtype, post_ln, untied):
    # embedding -> (ln_f) -> head: head backward, then the embedding backward
    # on its dx; the tied token table gets both shares
    lib = _lib()
    cfg = synth.GPTConfig(vocab=300, ctx=48, n_embd=64, n_head=2, n_layer=0, n_ff=128, dtype=dtype,
                          post_ln=post_ln, untied=untied)
    params = synth.make_params(cfg, seed=5, cfg_id=32, init="stress")
    Pf = synth.unpack_f64(cfg, params)
    B, T = 3, 41
    idx = synth.make_ids(cfg, B, T, seed=5)
    x0 = (Pf["wte"][idx] + Pf["wpe"][:T]).reshape(B * T, -1).astype(np.float32)   # embedding output (input)
    P = lib.params_to_device(cfg, synth.pack(cfg, params))
    n = lib.param_count(cfg)
    grads = torch.zeros(n, dtype=torch.float32, device="cuda")
    dx = torch.empty((B * T, cfg.n_embd), dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.head_backward_workspace_bytes(cfg, B, T), dtype=torch.uint8, device="cuda")
    it = torch.from_numpy(idx.astype(np.int32)).cuda()
    lib.head_backward(cfg, P, it, torch.from_numpy(x0).cuda(), dx, grads, None, None, ws)
    lib.embedding_backward(cfg, it, dx, grads)
    torch.cuda.synchronize()
    g = grads.cpu().numpy().astype(np.float64)
    ref = G.grads_no_blocks(Pf, idx)
    tol = TOL[dtype]
    for nm in ("wte", "wpe", "lnf_g", "lnf_b", "head_w"):
        if nm not in ref:
            continue
        o, shape = _slot(lib, cfg, nm)
        got = g[o:o + int(np.prod(shape))].reshape(shape)
        lim = tol["s"] if nm.startswith("lnf") else tol["g"]
        assert _rel(got, ref[nm]) <= lim, (nm, _rel(got, ref[nm]))


def test_embedding_backward_matches_oracle_and_is_deterministic():
    lib = _lib()
    cfg = synth.GPTConfig(vocab=50, ctx=64, n_embd=200, n_head=2, n_layer=1, n_ff=400, dtype=synth.F32)
    rng = np.random.default_rng(12)
    B, T = 5, 60
    idx = rng.integers(0, 12, (B, T)).astype(np.int32)   # many repeats of few tokens
    idx[1, 4] = -1                                        # ids outside [0, V) contribute nothing
    idx[3, 0] = 50
    dx0 = rng.normal(0, 1, (B * T, cfg.n_embd)).astype(np.float32)
    n = lib.param_count(cfg)
    g0 = rng.normal(0, 1, n).astype(np.float32)
    outs = []
    for _ in range(2):
        grads = torch.from_numpy(g0).cuda()
        lib.embedding_backward(cfg, torch.from_numpy(idx).cuda(), torch.from_numpy(dx0).cuda(), grads)
        torch.cuda.synchronize()
        outs.append(grads.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])
    keep = (idx >= 0) & (idx < cfg.vocab)
    # token rows: only positions with an id in [0, V); position rows: every position
    dE, _ = G.embedding_backward(np.where(keep, idx, 0), np.where(keep[..., None], dx0.reshape(B, T, -1), 0.0)
                                 .astype(np.float64), cfg.vocab, cfg.ctx)
    _, dP = G.embedding_backward(np.zeros_like(idx), dx0.reshape(B, T, -1).astype(np.float64), cfg.vocab, cfg.ctx)
    got = outs[0].astype(np.float64) - g0
    o, _ = _slot(lib, cfg, "wte")
    np.testing.assert_allclose(got[o:o + cfg.vocab * cfg.n_embd].reshape(cfg.vocab, -1), dE, rtol=1e-5, atol=1e-5)
    o, _ = _slot(lib, cfg, "wpe")
    np.testing.assert_allclose(got[o:o + cfg.ctx * cfg.n_embd].reshape(cfg.ctx, -1), dP, rtol=1e-5, atol=1e-5)
    assert np.all(got[cfg.vocab * cfg.n_embd + cfg.ctx * cfg.n_embd:] == 0)


def test_gpt2_vocab_rows_in_full():
    # the GPT-2 head (V = 50257, C = 768) on 256 rows, bf16: every output compared
    lib = _lib()
    cfg = dc.replace(synth.GPT2, n_layer=1)
    params = synth.make_params(cfg, seed=3, cfg_id=33, init="bench")
    Pf = synth.unpack_f64(cfg, params)
    B, T = 2, 128
    idx = synth.make_ids(cfg, B, T, seed=3)
    x = np.random.default_rng(3).normal(0, 1.0, (B * T, cfg.n_embd)).astype(np.float32)
    dx, dg, loss = _run_head_backward(lib, cfg, params, idx, x)
    ref = G.head_backward(Pf, x.astype(np.float64), O.derived_targets(idx).reshape(-1))
    assert _rel(dx, ref["dx"]) <= TOL[synth.BF16]["g"]
    o, _ = _slot(lib, cfg, "wte")
    assert _rel(dg[o:o + cfg.vocab * cfg.n_embd].reshape(cfg.vocab, -1), ref["head"]) <= TOL[synth.BF16]["g"]
    assert abs(loss - ref["loss"]) <= 1e-2 * abs(ref["loss"])


def test_gpt2_bench_shape_sampled():
    # B = 8, T = 1024, bf16, as timed: sampled dx rows (each needs only its own
    # logits row) and sampled head-gradient rows (each needs every row's
    # log-sum-exp, computed in fp64 chunks)
    lib = _lib()
    cfg = synth.GPT2
    params = synth.make_params(cfg, seed=0, cfg_id=34, init="bench")
    Pf = synth.unpack_f64(cfg, params)
    B, T = 8, 1024
    idx = synth.make_ids(cfg, B, T, seed=0)
    x = np.random.default_rng(0).normal(0, 1.0, (B * T, cfg.n_embd)).astype(np.float32)
    dx, dg, loss = _run_head_backward(lib, cfg, params, idx, x)
    y = O.derived_targets(idx).reshape(-1)
    n_valid = int((y >= 0).sum())
    E = Pf["wte"]
    a = O.layer_norm(x.astype(np.float64), Pf["lnf_g"], Pf["lnf_b"])
    rows = [0, 1023, 1024, 4097, 8191]
    for r in rows:
        if y[r] < 0:                      # last position of a sequence: no target, no gradient
            assert np.all(dx[r] == 0)
            continue
        hb = G.head_backward(Pf, x[r:r + 1].astype(np.float64), y[r:r + 1])
        want = hb["dx"][0] / n_valid      # the row alone has n_valid 1; dx is linear in dz
        assert _rel(dx[r], want) <= TOL[synth.BF16]["g"], (r, _rel(dx[r], want))
    lse = np.empty(B * T)
    for r0 in range(0, B * T, 512):
        z = a[r0:r0 + 512] @ E.T
        m = z.max(axis=1)
        lse[r0:r0 + 512] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    o, _ = _slot(lib, cfg, "wte")
    W = dg[o:o + cfg.vocab * cfg.n_embd].reshape(cfg.vocab, -1)
    valid = y >= 0
    for v in [0, 198, 13, 50256, 31000]:
        dzv = np.exp(a @ E[v] - lse) - (y == v)
        dzv[~valid] = 0.0
        want = (dzv / n_valid) @ a
        assert _rel(W[v], want) <= TOL[synth.BF16]["g"], (v, _rel(W[v], want))
    zy = np.einsum("nc,nc->n", a[valid], E[y[valid]])
    loss_ref = float((lse[valid] - zy).mean())
    assert abs(loss - loss_ref) <= 1e-2 * abs(loss_ref)
