"""Vocabulary shards on one GPU: the output weight cut into uneven row ranges,
each shard's forward, the merge of the per-row (lse, target logit) pairs, and
each shard's backward with the merged lse -- summed dX partials and
concatenated dW rows -- against the float64 oracle of the unsharded problem."""
import numpy as np
import pytest
import torch

import lm_head_linear_flce_amd as F
import oracle
import synth
from gpu_util import DEV, LSE_ABS, TOL, to_device

pytestmark = pytest.mark.gpu


def _cuts(V, shards):
    # uneven, not on tile boundaries
    c = [0] + [int(V * (k + 0.37) / shards) for k in range(1, shards)] + [V]
    return list(zip(c[:-1], c[1:]))


@pytest.mark.parametrize("name,ov,shards,reduction", [
    ("qwen2_7b_head", dict(T=777, H=512, V=5003, seed=211), 3, None),
    ("ragged_vocab", dict(T=1031, H=128, V=4099, seed=212), 2, None),
    ("tiny_f32", {}, 4, None),
    ("qwen3_sft_batch", dict(T=613, H=392, V=5003, seed=213), 3, "none"),
])
def test_vocab_shards_equal_the_whole(name, ov, shards, reduction):
    w = synth.workload(name, **ov)
    red = reduction or w.reduction
    g = np.random.default_rng(7).standard_normal(w.N) if red == "none" else 1.0
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index, reduction=red,
                      shift=w.shift, grad_scale=g, mode="rows", chunk=1024)
    X, W, lab = to_device(w)
    parts = _cuts(w.V, shards)
    lses, zts = [], []
    for v0, v1 in parts:
        lse_s, zt_s, st = F.shard_forward(X, W[v0:v1].contiguous(), lab, v0, w.V,
                                          ignore_index=w.ignore_index, shift=w.shift)
        lses.append(lse_s)
        zts.append(zt_s)
    loss, lse, n_valid, st = F.shard_merge(torch.stack(lses), torch.stack(zts), lab, w.V,
                                           ignore_index=w.ignore_index, shift=w.shift,
                                           reduction=red)
    gs = torch.tensor(g, dtype=torch.float32, device=DEV) if red == "none" else None
    dX32 = torch.zeros((w.N, w.H), dtype=torch.float32, device=DEV)
    dWs = []
    for v0, v1 in parts:
        dXp, dW_s, bst = F.shard_backward(X, W[v0:v1].contiguous(), lab, lse, v0, w.V,
                                          grad_scale=gs, ignore_index=w.ignore_index,
                                          shift=w.shift, reduction=red)
        dX32 += dXp.reshape(w.N, w.H)           # stands in for the FP32 all-reduce
        dWs.append(dW_s)
    torch.cuda.synchronize()
    assert int(st) == 0 and int(bst) == 0 and int(n_valid) == ref["n_valid"]
    tol = TOL[w.dtype]
    _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    got_lse = lse.double().cpu().numpy()
    assert np.abs(got_lse[valid] - ref["lse"][valid]).max() <= LSE_ABS
    assert np.all(got_lse[~valid] == 0.0)
    if red == "none":
        gl = loss.double().cpu().numpy()
        assert np.abs(gl - ref["loss"]).max() <= LSE_ABS + tol["loss_rel"] * np.abs(ref["loss"]).max()
    else:
        assert abs(float(loss) - ref["loss"]) <= tol["loss_rel"] * abs(ref["loss"])
    dX = dX32.to(X.dtype).double().cpu().numpy()          # one rounding after the sum
    dW = torch.cat(dWs).double().cpu().numpy()
    for nm, gt, r in (("dX", dX, ref["dX"]), ("dW", dW, ref["dW"])):
        assert oracle.cosine(gt, r) >= tol["cos"], nm
        if tol["maxabs"] is not None:
            assert np.abs(gt - r).max() <= tol["maxabs"] * np.abs(r).max(), nm


def test_single_shard_is_the_plain_forward():
    w = synth.workload("qwen2_7b_head", T=500, H=256, V=3001, seed=214)
    X, W, lab = to_device(w)
    loss, lse, _, _ = F.forward(X, W, lab, w.ignore_index, w.shift, w.reduction)
    lse_s, zt_s, _ = F.shard_forward(X, W, lab, 0, w.V, ignore_index=w.ignore_index,
                                     shift=w.shift)
    loss2, lse2, _, _ = F.shard_merge(lse_s[None], zt_s[None], lab, w.V,
                                      ignore_index=w.ignore_index, shift=w.shift,
                                      reduction=w.reduction)
    torch.cuda.synchronize()
    assert torch.equal(lse_s, lse)
    assert abs(float(loss2) - float(loss)) <= 1e-6 * abs(float(loss))


def test_eight_shards_full_size_against_stored_oracle():
    """The full Qwen2-7B-like head cut into 8 uneven vocabulary shards (the
    per-device share of an 8-way column-parallel output layer, ~19K rows
    each): the merged loss and every row's lse against the stored float64
    values, the summed FP32 dX partials (one rounding) and the concatenated
    shard dW rows on the stored sampled rows."""
    import os
    from gpu_util import check_sampled_rows
    from test_gpu_parity import GOLDEN
    path = os.path.join(GOLDEN, "full_qwen2_7b_head.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_full_expected.py)")
    e = np.load(path)
    w = synth.workload("qwen2_7b_head")
    print("[shards full] 8 shards", flush=True)
    X, W, lab = to_device(w)
    parts = _cuts(w.V, 8)
    lses, zts = [], []
    for v0, v1 in parts:
        lse_s, zt_s, st = F.shard_forward(X, W[v0:v1], lab, v0, w.V,
                                          ignore_index=w.ignore_index, shift=w.shift)
        assert int(st) == 0
        lses.append(lse_s)
        zts.append(zt_s)
    loss, lse, n_valid, st = F.shard_merge(torch.stack(lses), torch.stack(zts), lab, w.V,
                                           ignore_index=w.ignore_index, shift=w.shift,
                                           reduction=w.reduction)
    dX32 = torch.zeros((w.N, w.H), dtype=torch.float32, device=DEV)
    dWs = []
    for v0, v1 in parts:
        dXp, dW_s, bst = F.shard_backward(X, W[v0:v1], lab, lse, v0, w.V,
                                          ignore_index=w.ignore_index, shift=w.shift,
                                          reduction=w.reduction)
        assert int(bst) == 0
        dX32 += dXp.reshape(w.N, w.H)
        dWs.append(dW_s)
    torch.cuda.synchronize()
    assert int(st) == 0 and int(n_valid) == int(e["n_valid"])
    tol = TOL[w.dtype]
    _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    got_lse = lse.double().cpu().numpy()
    assert np.abs(got_lse[valid] - e["lse"][valid]).max() <= LSE_ABS
    assert np.all(got_lse[~valid] == 0.0)
    assert abs(float(loss) - float(e["loss"])) <= tol["loss_rel"] * abs(float(e["loss"]))
    got = dict(dX=dX32.to(X.dtype).double().cpu().numpy(),
               dW=torch.cat(dWs).double().cpu().numpy())
    check_sampled_rows(w, got, e, what="8 shards")
    assert np.all(got["dX"][~valid] == 0.0)
