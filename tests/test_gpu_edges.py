"""Degenerate shapes against the float64 oracle, in both modes: one row, the
narrowest hidden size the ABI allows (H = 8: one 16-byte bf16 chunk, a single
K step that is mostly tail), a one- and a two-entry vocabulary, a vocabulary
one past a tile, and a handful of one-token sequences under shift."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check, run, run_chunked

pytestmark = pytest.mark.gpu

CASES = [
    # B, T, H, V, dtype, shift, reduction, ignored rows
    (1, 1, 8, 1, "f32", False, "mean", 0),
    (1, 1, 8, 1, "bf16", False, "sum", 0),
    (2, 3, 8, 2, "f32", True, "mean", 0),
    (1, 5, 16, 257, "bf16", False, "sum", 2),
    (1, 300, 8, 300, "bf16", False, "mean", 30),
    (3, 1, 24, 513, "f32", False, "mean", 0),
    (4, 2, 40, 1000, "bf16", True, "mean", 1),
]


def _ids(c):
    B, T, H, V, dt, sh, red, ign = c
    return f"B{B}-T{T}-H{H}-V{V}-{dt}-{'shift' if sh else 'noshift'}-{red}-ign{ign}"


@pytest.mark.parametrize("mode", ["recompute", "chunked"])
@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_degenerate_shapes(case, mode):
    B, T, H, V, dt, sh, red, ign = case
    w = synth.make_workload("edge", B=B, T=T, H=H, V=V, dtype=dt, seed=7000 + B * T + V,
                            mask="count" if ign else None, mask_arg=ign or None,
                            shift=sh, reduction=red)
    print(f"[edge] {mode} {_ids(case)}", flush=True)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="global")
    got = run(w) if mode == "recompute" else run_chunked(w)
    if V == 1:
        # one entry: softmax is 1, every valid row's loss and gradient vanish
        # and lse is the logit itself
        assert got["status"] == 0 and got["n_valid"] == ref["n_valid"]
        assert abs(got["loss"]) <= 1e-6
        _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
        assert np.abs(got["lse"][valid] - ref["lse"][valid]).max() <= 1e-4
        assert np.abs(got["dX"]).max() <= 1e-6 and np.abs(got["dW"]).max() <= 1e-6
        return
    check(w, got, ref, what=f"{mode} {_ids(case)}")
    _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    assert np.all(got["dX"][~valid] == 0.0)
