"""GPU parity of the block backward (gpt_block_backward) and of the whole
gradient chain (gpt_forward_train -> gpt_head_backward -> gpt_block_backward
for each block in reverse -> gpt_embedding_backward) against the fp64
backward oracle, on the same inputs.

Tolerances (max |GPU - oracle| over max |oracle|, per tensor): fp32 1e-5
(fp32 products, and the attention gradient computed in fp32 from recomputed
probabilities: measured at most 8e-7); bf16 2e-2 (the recomputed
activations a1, q, k, u, o, u_fc, h and the gradients fed to the products
are rounded to bf16, 2^-9 relative each, about six such roundings on every
path: measured at most 6.6e-3; the test prints every tensor's error).
"""
import dataclasses as dc

import numpy as np
import pytest

from decoder_only_transformer_attn_amd import synth
from oracle import grad_oracle as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = {synth.F32: 1e-5, synth.BF16: 2e-2}


def _lib():
    from decoder_only_transformer_attn_amd import lib
    lib.load()
    return lib


def _rel(got, ref):
    return float(np.abs(np.asarray(got, np.float64) - ref).max() / max(np.abs(ref).max(), 1e-30))


def _slot(cfg, name):
    for nm, shape, off in synth.blob_layout(cfg):
        if nm == name:
            return off, shape
    raise KeyError(name)


def run_block(cfg, params, layer, x, dy, seed=0):
    lib = _lib()
    B, T, C = x.shape
    P = lib.params_to_device(cfg, synth.pack(cfg, params))
    n = lib.param_count(cfg)
    g0 = np.random.default_rng(seed).normal(0, 1e-3, n).astype(np.float32)
    grads = torch.from_numpy(g0).cuda()
    xd = torch.from_numpy(x.reshape(B * T, C).astype(np.float32)).cuda()
    dyd = torch.from_numpy(dy.reshape(B * T, C).astype(np.float32)).cuda()
    dx = torch.full_like(xd, float("nan"))
    # workspace filled with 0xFF bytes (NaN in bf16 and fp32): a read of any
    # byte no kernel of the call wrote shows up as a non-finite gradient
    ws = torch.full((lib.block_backward_workspace_bytes(cfg, B, T),), 255, dtype=torch.uint8, device="cuda")
    lib.block_backward(cfg, P, layer, B, T, xd, dyd, dx, grads, ws)
    torch.cuda.synchronize()
    return dx.cpu().numpy().reshape(B, T, C), grads.cpu().numpy().astype(np.float64) - g0


def check_block(cfg, layer, B, T, seed, init="stress"):
    params = synth.make_params(cfg, seed=seed, cfg_id=71, init=init)
    Pf = synth.unpack_f64(cfg, params)
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1.0, (B, T, cfg.n_embd)).astype(np.float32)
    dy = rng.normal(0, 1e-3, (B, T, cfg.n_embd)).astype(np.float32)
    dx, dg = run_block(cfg, params, layer, x, dy, seed)
    ref_dx, ref_g = G.block_backward(x.astype(np.float64), Pf["layers"][layer], dy.astype(np.float64), cfg.n_head,
                                     cfg.ln_eps, Pf["act"])
    tol = TOL[cfg.dtype]
    errs = {"dx": _rel(dx, ref_dx)}
    touched = np.zeros(dg.shape, bool)
    for key, ref in ref_g.items():
        off, shape = _slot(cfg, f"h{layer}.{key}")
        n = int(np.prod(shape))
        errs[key] = _rel(dg[off:off + n].reshape(shape), ref)
        touched[off:off + n] = True
    print({k: f"{v:.2e}" for k, v in errs.items()})
    assert np.isfinite(dx).all()
    assert np.isfinite(dg).all()
    for k, v in errs.items():
        assert v <= tol, (k, v)
    assert np.all(dg[~touched] == 0)   # no other tensor's gradient changed


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("B,T", [(2, 37), (1, 64)])
def test_block_backward_matches_oracle(dtype, act, B, T):
    cfg = synth.GPTConfig(vocab=97, ctx=64, n_embd=64, n_head=2, n_layer=2, n_ff=128, dtype=dtype, act=act)
    check_block(cfg, 1, B, T, seed=B * T + act)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("C,H", [(256, 4), (512, 8), (1024, 16)])
def test_block_backward_register_row_widths(dtype, C, H):
    # widths of 256, 512 and 1024 columns: the LayerNorm backward holds one,
    # two or four 16-byte pieces of each row per lane
    cfg = synth.GPTConfig(vocab=97, ctx=64, n_embd=C, n_head=H, n_layer=1, n_ff=2 * C, dtype=dtype)
    check_block(cfg, 0, 1, 40, seed=C + H)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("T", [100, 60, 128])
def test_block_backward_head_width_128(dtype, T):
    # D = 128 with 64 < T < 128: the contractions of the attention backward
    # take 128-row tiles, so the score tiles they read must be 128 x 128 too
    # (64 x 64 score tiles leave the tile above the diagonal unwritten)
    cfg = synth.GPTConfig(vocab=97, ctx=128, n_embd=256, n_head=2, n_layer=1, n_ff=512, dtype=dtype)
    check_block(cfg, 0, 2, T, seed=T + 128)


def test_block_backward_gpt2_width_bf16():
    cfg = dc.replace(synth.GPT2, n_layer=1)
    check_block(cfg, 0, 1, 256, seed=5, init="bench")


def test_block_backward_gpt2_width_long_ragged_sequence_bf16():
    # 1000 positions: score tiles of 128 x 128 with a padded last row / column tile
    cfg = dc.replace(synth.GPT2, n_layer=1)
    check_block(cfg, 0, 1, 1000, seed=6, init="bench")


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_full_gradient_chain_matches_oracle(dtype):
    lib = _lib()
    cfg = synth.GPTConfig(vocab=300, ctx=48, n_embd=64, n_head=2, n_layer=2, n_ff=128, dtype=dtype)
    params = synth.make_params(cfg, seed=8, cfg_id=72, init="stress")
    Pf = synth.unpack_f64(cfg, params)
    B, T = 2, 33
    idx = synth.make_ids(cfg, B, T, seed=8)
    P = lib.params_to_device(cfg, synth.pack(cfg, params))
    grads = torch.zeros(lib.param_count(cfg), dtype=torch.float32, device="cuda")
    loss = lib.gradients(cfg, P, torch.from_numpy(idx).cuda(), grads)
    torch.cuda.synchronize()
    g = grads.cpu().numpy().astype(np.float64)
    ref = G.grads_full(Pf, idx, cfg.n_head)
    tol = TOL[dtype]
    assert abs(float(loss.item()) - ref["loss"]) <= (1e-4 if dtype == synth.F32 else 1e-2) * abs(ref["loss"])
    errs = {}
    for nm in ("wte", "wpe", "lnf_g", "lnf_b"):
        o, shape = _slot(cfg, nm)
        errs[nm] = _rel(g[o:o + int(np.prod(shape))].reshape(shape), ref[nm])
    for l in range(cfg.n_layer):
        for key, r in ref["layers"][l].items():
            o, shape = _slot(cfg, f"h{l}.{key}")
            errs[f"{l}.{key}"] = _rel(g[o:o + int(np.prod(shape))].reshape(shape), r)
    print({k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= tol, (k, v)


def test_block_backward_is_deterministic():
    cfg = synth.GPTConfig(vocab=97, ctx=64, n_embd=64, n_head=2, n_layer=1, n_ff=128, dtype=synth.BF16)
    params = synth.make_params(cfg, seed=2, cfg_id=73, init="stress")
    rng = np.random.default_rng(2)
    x = rng.normal(0, 1, (2, 50, 64)).astype(np.float32)
    dy = rng.normal(0, 1e-3, x.shape).astype(np.float32)
    a = run_block(cfg, params, 0, x, dy)
    b = run_block(cfg, params, 0, x, dy)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_forward_train_without_loss_writes_the_same_residuals():
    # a null mean_loss skips the head: the residual streams must not change
    lib = _lib()
    cfg = synth.GPTConfig(vocab=300, ctx=48, n_embd=64, n_head=2, n_layer=2, n_ff=128, dtype=synth.BF16)
    params = synth.make_params(cfg, seed=9, cfg_id=74, init="stress")
    P = lib.params_to_device(cfg, synth.pack(cfg, params))
    B, T = 2, 33
    idx = torch.from_numpy(synth.make_ids(cfg, B, T, seed=9)).cuda()
    ws = torch.empty(lib.workspace_bytes(cfg, B, T), dtype=torch.uint8, device="cuda")
    xs = [torch.full((cfg.n_layer + 1, B * T, cfg.n_embd), float("nan"), device="cuda") for _ in range(2)]
    loss = torch.full((1,), float("nan"), device="cuda")
    lib.forward_train(cfg, P, idx, xs[0], ws, None, loss)
    lib.forward_train(cfg, P, idx, xs[1], ws, None, None)
    torch.cuda.synchronize()
    assert torch.isfinite(loss).all()
    assert torch.equal(xs[0], xs[1])
