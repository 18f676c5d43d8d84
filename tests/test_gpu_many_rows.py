"""Many rows: more than 2048 token tiles, so the forward runs one vocabulary
range per token tile over a grid rounded up to a multiple of 8 workgroups, and
the token-tile count (2051) is not a multiple of 8.  Every token tile's first
and last row is checked against the float64 oracle (lse, dX), and all of dW."""
import numpy as np
import pytest
import torch

import lm_head_linear_flce_amd as F
import oracle
import synth
from gpu_util import DEV, LSE_ABS, TOL

pytestmark = pytest.mark.gpu


def test_more_than_2048_token_tiles():
    T, H, V = 525000, 64, 300
    w = synth.make_workload("many_rows", B=1, T=T, H=H, V=V, dtype="bf16", seed=7711,
                            labels="uniform", shift=False, reduction="mean")
    print(f"[many-rows] N={w.N} H={H} V={V} bf16", flush=True)
    X = torch.from_numpy(w.X).to(DEV).to(torch.bfloat16)
    W = torch.from_numpy(w.W).to(DEV).to(torch.bfloat16)
    lab = torch.from_numpy(w.labels).to(DEV)
    loss, lse, n_valid, status = F.forward(X, W, lab, w.ignore_index, w.shift, w.reduction)
    dX, dW, bstatus = F.backward(X, W, lab, lse, ignore_index=w.ignore_index, shift=w.shift,
                                 reduction=w.reduction)
    torch.cuda.synchronize()
    assert int(status) == 0 and int(bstatus) == 0 and int(n_valid) == w.N
    tiles = (w.N + 255) // 256
    assert tiles == 2051
    rows = np.unique(np.concatenate([np.arange(tiles) * 256,
                                     np.minimum(np.arange(tiles) * 256 + 255, w.N - 1)]))
    ref = oracle.forward_rows(w.X, w.W, w.labels, rows=rows)
    got_lse = lse.double().cpu().numpy()
    err = np.abs(got_lse[rows] - ref["lse"][rows]).max()
    assert err <= LSE_ABS, f"lse max abs err {err}"
    full = oracle.forward_rows(w.X, w.W, w.labels)
    assert abs(float(loss) - full["loss"]) <= TOL["bf16"]["loss_rel"] * abs(full["loss"])
    c = 1.0 / w.N
    rdx = oracle.dx_rows(w.X, w.W, full["y"], full["valid"], full["lse"], c, rows)
    gdx = dX.double().cpu().numpy()[rows]
    assert oracle.cosine(gdx, rdx) >= TOL["bf16"]["cos"]
    assert np.abs(gdx - rdx).max() <= TOL["bf16"]["maxabs"] * np.abs(rdx).max()
    rdw = oracle.dw_rows(w.X, w.W, full["y"], full["valid"], full["lse"], c, np.arange(V))
    gdw = dW.double().cpu().numpy()
    assert oracle.cosine(gdw, rdw) >= TOL["bf16"]["cos"]
    assert np.abs(gdw - rdw).max() <= TOL["bf16"]["maxabs"] * np.abs(rdw).max()


def _long_rows_case(T, H, V, seed):
    """Sampled lse and dX rows (every 64th token tile's edges) and all of dW
    (small V) against the oracle for one long sequence."""
    w = synth.make_workload("long_rows", B=1, T=T, H=H, V=V, dtype="bf16", seed=seed,
                            x_rms=True, labels="zipf", mask="prefix", mask_arg=4096,
                            shift=True, reduction="mean")
    print(f"[long-rows] N={w.N} H={H} V={V} bf16", flush=True)
    X = torch.from_numpy(w.X).to(DEV).to(torch.bfloat16)
    W = torch.from_numpy(w.W).to(DEV).to(torch.bfloat16)
    lab = torch.from_numpy(w.labels).to(DEV)
    loss, lse, n_valid, status = F.forward(X, W, lab, w.ignore_index, w.shift, w.reduction)
    dX, dW, bstatus = F.backward(X, W, lab, lse, ignore_index=w.ignore_index, shift=w.shift,
                                 reduction=w.reduction)
    torch.cuda.synchronize()
    assert int(status) == 0 and int(bstatus) == 0
    full = oracle.forward_rows(w.X, w.W, w.labels, ignore_index=w.ignore_index, shift=True,
                               chunk=4096)
    assert int(n_valid) == full["n_valid"]
    assert abs(float(loss) - full["loss"]) <= TOL["bf16"]["loss_rel"] * abs(full["loss"])
    vrows = np.flatnonzero(full["valid"])
    edges = np.arange(0, len(vrows), 64 * 256)
    rows = np.unique(np.concatenate([vrows[edges], vrows[np.maximum(edges - 1, 0)],
                                     vrows[-2:], [0, w.N - 1]]))
    got_lse = lse.double().cpu().numpy()
    sel = rows[full["valid"][rows]]
    assert np.abs(got_lse[sel] - full["lse"][sel]).max() <= LSE_ABS
    c = 1.0 / full["n_valid"]
    rdx = oracle.dx_rows(w.X, w.W, full["y"], full["valid"], full["lse"], c, rows)
    gdx = dX.double().cpu().numpy()[rows]
    assert oracle.cosine(gdx, rdx) >= TOL["bf16"]["cos"]
    assert np.abs(gdx - rdx).max() <= TOL["bf16"]["maxabs"] * np.abs(rdx).max()
    rdw = oracle.dw_rows(w.X, w.W, full["y"], full["valid"], full["lse"], c, np.arange(V))
    gdw = dW.double().cpu().numpy()
    assert oracle.cosine(gdw, rdw) >= TOL["bf16"]["cos"]
    assert np.abs(gdw - rdw).max() <= TOL["bf16"]["maxabs"] * np.abs(rdw).max()


def test_rows_times_hidden_past_2_29():
    """N * H = 2^29 (262144 rows of H = 2048, 1 GiB of bf16 hidden states): the
    FP32 dX sums (2 GiB) and the one-hot row sums pass 2^31 bytes and the dW
    contraction runs over 0.5 Gi elements of X."""
    _long_rows_case(262144, 2048, 333, 7721)


def test_rows_times_hidden_past_2_30():
    """N * H just past 2^30 (532480 rows of H = 2048, 2.03 GiB of bf16 hidden
    states; 528383 valid rows): the dW tiles' K loop over the rows reaches past
    2^31 bytes of X, so their loaders rebase the buffer descriptor at every K
    step."""
    _long_rows_case(532480, 2048, 97, 7723)
