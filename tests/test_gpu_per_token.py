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
