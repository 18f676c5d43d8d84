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


def test_vocabulary_past_2_24_weight_past_2_31_bytes():
    """V = 2^24 + 43 at H = 64: W holds 2.1 GB of bf16 (past 2^31 bytes), the
    forward walks 65537 vocabulary tiles per token tile, the backward 33
    launches of 2^19-column blocks, and dW is written past 2^31 bytes.  Every
    valid row's lse, the loss, sampled dX rows and dW rows at the ends of the
    vocabulary, around 2^24 and on block edges, against the float64 oracle.
    (The chunked mode refuses this shape: one 256-row chunk of the softmax
    slab would pass 2^31 bytes.)"""
    T, H, V = 256, 64, 2 ** 24 + 43
    w = synth.make_workload("huge_vocab", B=1, T=T, H=H, V=V, dtype="bf16", seed=7733,
                            labels="uniform", mask="count", mask_arg=21, shift=False,
                            reduction="mean")
    print(f"[huge-vocab] N={w.N} H={H} V={V} bf16", flush=True)
    X = torch.from_numpy(w.X).to(DEV).to(torch.bfloat16)
    W = torch.from_numpy(w.W).to(DEV).to(torch.bfloat16)
    lab = torch.from_numpy(w.labels).to(DEV)
    loss, lse, n_valid, status = F.forward(X, W, lab, w.ignore_index, w.shift, w.reduction)
    dX, dW, bstatus = F.backward(X, W, lab, lse, ignore_index=w.ignore_index, shift=w.shift,
                                 reduction=w.reduction)
    torch.cuda.synchronize()
    y, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    n = int(valid.sum())
    assert int(status) == 0 and int(bstatus) == 0 and int(n_valid) == n
    # the whole-vocabulary logits of 16 rows at a time (2.1 GB of float64)
    ref = oracle.forward_rows(w.X, w.W, w.labels, ignore_index=w.ignore_index, chunk=16)
    got_lse = lse.double().cpu().numpy()
    assert np.abs(got_lse[valid] - ref["lse"][valid]).max() <= LSE_ABS
    assert np.all(got_lse[~valid] == 0.0)
    assert abs(float(loss) - ref["loss"]) <= TOL["bf16"]["loss_rel"] * abs(ref["loss"])
    c = 1.0 / n
    xrows = np.concatenate([np.flatnonzero(valid)[[0, 1, n // 2, n - 1]],
                            np.flatnonzero(~valid)[:2]])
    want_x = oracle.dx_rows(w.X, w.W, y, valid, ref["lse"], c, xrows)
    got_x = dX.reshape(w.N, H)[torch.from_numpy(xrows).to(DEV)].double().cpu().numpy()
    block = 1 << 19
    vids = np.unique(np.concatenate([
        [0, 1, 255, 256, block - 1, block, 2 ** 24 - 1, 2 ** 24, 2 ** 24 + 1, V - 2, V - 1],
        y[valid][:6]]))
    want_w = oracle.dw_rows(w.X, w.W, y, valid, ref["lse"], c, vids)
    got_w = dW[torch.from_numpy(vids).to(DEV)].double().cpu().numpy()
    for name, got, want in (("dX", got_x, want_x), ("dW", got_w, want_w)):
        for q in range(len(want)):
            if not np.any(want[q]):
                assert not np.any(got[q]), (name, q)
                continue
            assert oracle.cosine(got[q], want[q]) >= 0.999, (name, q)
            assert np.abs(got[q] - want[q]).max() <= 1e-2 * np.abs(want[q]).max(), (name, q)


def test_rows_at_the_softmax_slab_bound():
    """N = 2^22 - 256 rows at H = 8: the narrowest vocabulary block (256
    columns) of the softmax slab then spans 2^31 - 131072 bytes, the last
    slab offset before the 32-bit bound the plan enforces (one more token
    tile is FLCE_ERR_SHAPE), and the dW tiles' K loop over 4 million rows runs
    with per-step descriptors."""
    _long_rows_case(2 ** 22 - 256, 8, 300, 7725)
