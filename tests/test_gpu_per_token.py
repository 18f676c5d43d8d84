"""Per-token outputs (reduction "none"): per-row losses from the forward and a
per-row upstream gradient in the backward, against the float64 oracle."""
import numpy as np
import pytest
import torch

import lm_head_linear_flce_amd as F
import oracle
import synth
from gpu_util import DEV, LSE_ABS, TOL, to_device

pytestmark = pytest.mark.gpu

CASES = [("tiny_f32", {}), ("qwen2_7b_head", dict(T=777, H=512, V=3001, seed=21)),
         ("ragged_vocab", dict(T=1031, H=128, V=4099, seed=51))]


def _check_rows(w, got_loss, got_dX, got_dW, ref):
    tol = TOL[w.dtype]
    _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    want = ref["loss"]
    # per-row loss = lse - z_y: the lse bound plus the target logit's rounding
    err = np.abs(got_loss - want)
    assert err[valid].max() <= LSE_ABS + tol["loss_rel"] * np.abs(want[valid]).max()
    assert np.all(got_loss[~valid] == 0.0)
    for name, g, r in (("dX", got_dX, ref["dX"]), ("dW", got_dW, ref["dW"])):
        assert oracle.cosine(g, r) >= tol["cos"], name
        if tol["maxabs"] is not None:
            assert np.abs(g - r).max() <= tol["maxabs"] * np.abs(r).max(), name


@pytest.mark.parametrize("name,ov", CASES)
@pytest.mark.parametrize("mode", ["recompute", "chunked"])
def test_per_token_losses_and_gradients(name, ov, mode):
    w = synth.workload(name, **ov)
    g = np.random.default_rng(5).standard_normal(w.N)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index, reduction="none",
                      shift=w.shift, grad_scale=g, mode="rows", chunk=1024)
    X, W, lab = to_device(w)
    gs = torch.tensor(g, dtype=torch.float32, device=DEV)
    if mode == "recompute":
        loss, lse, _, st = F.forward(X, W, lab, w.ignore_index, w.shift, "none")
        dX, dW, bst = F.backward(X, W, lab, lse, grad_scale=gs, ignore_index=w.ignore_index,
                                 shift=w.shift, reduction="none")
        assert int(bst) == 0
    else:
        loss, lse, _, dX, dW, st = F.chunked(X, W, lab, grad_scale=gs,
                                             ignore_index=w.ignore_index, shift=w.shift,
                                             reduction="none")
    torch.cuda.synchronize()
    assert int(st) == 0 and loss.shape == (w.N,)
    _check_rows(w, loss.double().cpu().numpy(), dX.reshape(w.N, w.H).double().cpu().numpy(),
                dW.double().cpu().numpy(), ref)


def test_per_token_autograd():
    w = synth.workload("qwen2_7b_head", T=300, H=128, V=700, seed=171)
    X, W, lab = to_device(w)
    Xr = X.detach().clone().requires_grad_(True)
    Wr = W.detach().clone().requires_grad_(True)
    tok = F.linear_cross_entropy(Xr, Wr, lab, shift=True, reduction="none")
    assert tok.shape == lab.shape
    g = np.random.default_rng(6).standard_normal(w.N)
    (tok * torch.tensor(g, dtype=torch.float32, device=DEV).reshape(lab.shape)).sum().backward()
    ref = oracle.flce(w.X, w.W, w.labels, shift=True, reduction="none", grad_scale=g)
    assert oracle.cosine(Xr.grad.reshape(w.N, w.H).double().cpu().numpy(), ref["dX"]) >= 0.9999
    assert oracle.cosine(Wr.grad.double().cpu().numpy(), ref["dW"]) >= 0.9999
    # target log-probs are the negated per-token losses
    _, valid = oracle.targets(w.labels, True)
    lp = -tok.detach().reshape(-1).double().cpu().numpy()
    assert np.all(lp[valid] <= 1e-6) and np.all(lp[~valid] == 0.0)
    with pytest.raises(ValueError):
        F.linear_cross_entropy(Xr, Wr, lab, shift=True, reduction="none", mode="chunked")


def test_per_token_bad_label_is_nan():
    w = synth.workload("ragged_vocab", T=300, H=64, V=500, seed=121)
    w.labels[0, 5] = w.V + 3
    X, W, lab = to_device(w)
    loss, _, _, st = F.forward(X, W, lab, w.ignore_index, w.shift, "none")
    torch.cuda.synchronize()
    assert int(st) == F.FLCE_ERR_LABEL_RANGE and torch.isnan(loss).all()


@pytest.mark.parametrize("mode", ["recompute", "chunked"])
def test_per_token_full_size_against_stored_oracle(mode):
    """Reduction "none" at the full Qwen2-7B-like head (N = 8192, V = 152064):
    every valid row's loss against the stored float64 lse minus the row's
    target logit (a float64 dot product), and the stored dX rows scaled by the
    row's upstream gradient: dX_i = g_i (softmax - onehot)_i W, where the stored
    mean-reduction rows carry the factor grad_scale / n."""
    import os
    from test_gpu_parity import GOLDEN
    path = os.path.join(GOLDEN, "full_qwen2_7b_head.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_full_expected.py)")
    e = np.load(path)
    w = synth.workload("qwen2_7b_head")
    y, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    n, gs = int(e["n_valid"]), float(e["grad_scale"])
    assert n == int(valid.sum())
    rng = np.random.Generator(np.random.PCG64(4242))
    g = (rng.uniform(0.5, 1.5, size=w.N) * rng.choice([-1.0, 1.0], size=w.N)).astype(np.float32)
    print(f"[per-token full] {mode}", flush=True)
    X, W, lab = to_device(w)
    gt = torch.from_numpy(g).to(DEV)
    if mode == "recompute":
        loss, lse, _, st = F.forward(X, W, lab, w.ignore_index, w.shift, "none")
        dX, _, bst = F.backward(X, W, lab, lse, grad_scale=gt, ignore_index=w.ignore_index,
                                shift=w.shift, reduction="none")
    else:
        loss, _, _, dX, _, st = F.chunked(X, W, lab, grad_scale=gt, ignore_index=w.ignore_index,
                                          shift=w.shift, reduction="none")
        bst = st
    torch.cuda.synchronize()
    assert int(st) == 0 and int(bst) == 0
    got = loss.double().cpu().numpy().reshape(-1)
    zt = np.einsum("ij,ij->i", w.X[valid].astype(np.float64), w.W[y[valid]].astype(np.float64))
    want = np.zeros(w.N)
    want[valid] = e["lse"].astype(np.float64)[valid] - zt
    tol = TOL[w.dtype]
    err = np.abs(got - want)
    assert err[valid].max() <= LSE_ABS + tol["loss_rel"] * np.abs(want[valid]).max(), err.max()
    assert np.all(got[~valid] == 0.0)
    dXh = dX.reshape(w.N, w.H).double().cpu().numpy()
    for q, r in enumerate(e["dx_rows"]):
        b = e["dx"][q].astype(np.float64) * (float(g[r]) * n / gs)
        a = dXh[r]
        if not np.any(b):
            assert not np.any(a), f"dX row {r}"
            continue
        assert oracle.cosine(a, b) >= 0.999, f"dX row {r}"
        assert np.abs(a - b).max() <= 1e-2 * np.abs(b).max(), f"dX row {r}"
