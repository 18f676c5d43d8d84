"""Shared helpers of the GPU tests: run the HIP path through the binding on a
synthetic workload and compare with the float64 oracle."""
import numpy as np
import torch

import lm_head_linear_flce_amd as F
import oracle

DEV = "cuda:0"

# the tolerances of the build's contract, per input dtype
TOL = {
    "f32": dict(loss_rel=1e-5, cos=0.999999, maxabs=None),
    "bf16": dict(loss_rel=2e-3, cos=0.9999, maxabs=1e-2),
}
LSE_ABS = 1e-4     # per valid row, both dtypes


def to_device(w):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    X = torch.from_numpy(w.X).to(DEV).to(dt).reshape(w.B, w.T, w.H)
    W = torch.from_numpy(w.W).to(DEV).to(dt)
    lab = torch.from_numpy(np.ascontiguousarray(w.labels)).to(DEV)
    return X, W, lab


def run(w, grad_dtype=None, grad_scale=None, X=None, W=None, lab=None):
    if X is None:
        X, W, lab = to_device(w)
    loss, lse, n_valid, status = F.forward(X, W, lab, w.ignore_index, w.shift, w.reduction)
    gs = None if grad_scale is None else torch.tensor(grad_scale, dtype=torch.float32,
                                                        device=DEV)
    dX, dW, bstatus = F.backward(X, W, lab, lse, grad_scale=gs,
                                 ignore_index=w.ignore_index, shift=w.shift,
                                 reduction=w.reduction, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return dict(loss=float(loss), lse=lse.double().cpu().numpy(),
                n_valid=int(n_valid), status=int(status), bstatus=int(bstatus),
                dX=dX.reshape(w.N, w.H).double().cpu().numpy(),
                dW=dW.double().cpu().numpy())


def run_chunked(w, grad_dtype=None, grad_scale=None, chunk_rows=0):
    """The same outputs from one flce_chunked call."""
    X, W, lab = to_device(w)
    gs = None if grad_scale is None else torch.tensor(grad_scale, dtype=torch.float32,
                                                        device=DEV)
    loss, lse, n_valid, dX, dW, status = F.chunked(
        X, W, lab, grad_scale=gs, ignore_index=w.ignore_index, shift=w.shift,
        reduction=w.reduction, grad_dtype=grad_dtype, chunk_rows=chunk_rows)
    torch.cuda.synchronize()
    return dict(loss=float(loss), lse=lse.double().cpu().numpy(),
                n_valid=int(n_valid), status=int(status), bstatus=int(status),
                dX=dX.reshape(w.N, w.H).double().cpu().numpy(),
                dW=dW.double().cpu().numpy())


def check(w, got, ref, dx_rows=None, dw_rows=None, what="", lse_rel=0.0):
    """Contract tolerances plus the per-row lse diagnostic.  lse_rel widens the
    per-row lse bound by lse_rel * |lse| (for logits far from zero, where the
    FP32 sum over H alone carries errors of that size)."""
    tol = TOL[w.dtype]
    assert got["status"] == 0 and got["bstatus"] == 0, what
    assert got["n_valid"] == ref["n_valid"], what
    rl = abs(got["loss"] - ref["loss"]) / max(abs(ref["loss"]), 1e-30)
    assert rl <= tol["loss_rel"], f"{what} loss {got['loss']} vs {ref['loss']} rel {rl}"
    _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    if valid.any():
        err = np.abs(got["lse"][valid] - ref["lse"][valid])
        bound = LSE_ABS + lse_rel * np.abs(ref["lse"][valid])
        assert np.all(err <= bound), f"{what} lse max abs err {err.max()}"
    assert np.all(got["lse"][~valid] == 0.0), what
    gx = got["dX"] if dx_rows is None else got["dX"][dx_rows]
    gw = got["dW"] if dw_rows is None else got["dW"][dw_rows]
    out = {}
    for name, g, r in (("dX", gx, ref["dX"]), ("dW", gw, ref["dW"])):
        cos = oracle.cosine(g, r)
        assert cos >= tol["cos"], f"{what} {name} cosine {cos}"
        if tol["maxabs"] is not None:
            m = np.abs(g - r).max()
            assert m <= tol["maxabs"] * np.abs(r).max(), f"{what} {name} max abs {m}"
        out[name] = cos
    return out


def check_sampled_rows(w, got, e, what=""):
    """Each stored row on its own: cosine >= 0.999 and max-abs error within
    1e-2 of the row's largest value.  A dW row of a vocabulary entry that no
    row targets is pure softmax part, so a wrong vocabulary block or tile
    edge shows here even where the whole-sample cosine would hide it."""
    for name, rows, ref in (("dX", e["dx_rows"], e["dx"]), ("dW", e["dw_rows"], e["dw"])):
        g = got[name][rows]
        for q, r in enumerate(rows):
            a, b = g[q], ref[q].astype(np.float64)
            if not np.any(b):
                assert not np.any(a), f"{what} {name} row {r}"
                continue
            cos = oracle.cosine(a, b)
            assert cos >= 0.999, f"{what} {name} row {r} cosine {cos}"
            err = np.abs(a - b).max() / np.abs(b).max()
            assert err <= 1e-2, f"{what} {name} row {r} max-abs {err}"


def check_block_coverage(w, e):
    """Every vocabulary block of both backward widths stored with e holds at
    least two sampled dW rows (its first and last column)."""
    rows = set(int(r) for r in e["dw_rows"])
    for wdt in (int(x) for x in e["block_widths"]):
        for b0 in range(0, w.V, wdt):
            b1 = min(b0 + wdt, w.V) - 1
            assert b0 in rows and b1 in rows, (wdt, b0, b1)


def soft_parts(w, dX, dW, n):
    """The softmax parts of the gradients, P W and P^T X, rebuilt from dX and
    dW by removing the one-hot term: dX_i / c + W_{y_i} and dW / c + the sum
    of X_i over the rows whose target is v (mean: c = 1 / n)."""
    y, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    c = 1.0 / n if w.reduction == "mean" else 1.0
    X = w.X.reshape(w.N, w.H).astype(np.float64)
    Wt = w.W.astype(np.float64)
    sx = dX[valid] / c + Wt[y[valid]]
    sw = dW / c
    np.add.at(sw, y[valid], X[valid])
    return sx, sw


def soft_tolerance(w):
    """(minimum cosine, norm-ratio tolerance) of the softmax parts.  The slab
    that the contractions read holds only the softmax part c p (fp32, or
    bf16 with relative rounding 2^-9 per entry); the one-hot part is added in
    FP32 to the gradient sums.  With bf16 inputs the rebuilt soft parts then
    carry only that per-entry rounding noise plus the FP32 accumulation:
    cosine >= 0.999 and the norm within 0.5 %.  A
    missing or misplaced softmax term gives a cosine near 0, a wrong scale a
    norm ratio far from 1."""
    if w.dtype == "f32":
        return 0.99999, 1e-4
    return 0.999, 0.005
