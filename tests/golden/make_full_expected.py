"""Write the float64 oracle's expected values for the four full-size bf16
workloads (and the full tiny fp32 one) to tests/golden/full_<name>.npz.

Only ``synth`` (inputs) and ``oracle`` (arithmetic) are used.  Stored per
workload: n_valid, the loss, lse of every row, and dX / dW on sampled rows
(sampled dX rows include the first and last valid rows and an ignored row;
sampled dW rows include the most frequent targets, a target-free id and the
last vocabulary rows, which sit in the ragged last tile).

    python tests/golden/make_full_expected.py [name ...]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

N_DX = 12
N_DW = 12


def sample_rows(y, valid, seed):
    rng = np.random.default_rng(seed)
    vrows = np.flatnonzero(valid)
    pick = {int(vrows[0]), int(vrows[-1])}
    ign = np.flatnonzero(~valid)
    if len(ign):
        pick.add(int(ign[len(ign) // 2]))
    while len(pick) < N_DX:
        pick.add(int(rng.choice(vrows)))
    return np.array(sorted(pick))


def sample_vocab(y, valid, V, seed):
    rng = np.random.default_rng(seed)
    counts = np.bincount(y[valid], minlength=V)
    top = np.argsort(-counts, kind="stable")[:4]
    pick = {int(t) for t in top}
    absent = np.flatnonzero(counts == 0)
    if len(absent):
        pick.add(int(absent[0]))
    pick.update({V - 1, V - 2})
    while len(pick) < N_DW:
        pick.add(int(rng.integers(0, V)))
    return np.array(sorted(pick))


def make(name):
    t0 = time.time()
    w = synth.workload(name)
    f = oracle.forward_rows(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                            reduction=w.reduction, shift=w.shift, chunk=256)
    n = f["n_valid"]
    c = (1.0 / n) if w.reduction == "mean" else 1.0
    rows = sample_rows(f["y"], f["valid"], 7)
    vids = sample_vocab(f["y"], f["valid"], w.V, 8)
    dx = oracle.dx_rows(w.X, w.W, f["y"], f["valid"], f["lse"], c, rows)
    dw = oracle.dw_rows(w.X, w.W, f["y"], f["valid"], f["lse"], c, vids)
    out = os.path.join(HERE, f"full_{name}.npz")
    np.savez_compressed(out, n_valid=n, loss=f["loss"], lse=f["lse"],
                        dx_rows=rows, dx=dx, dw_rows=vids, dw=dw, grad_scale=1.0)
    print(f"{name}: n={n} loss={f['loss']:.10f} ({time.time() - t0:.1f}s) -> {out}",
          flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or list(synth.WORKLOADS)
    for nm in names:
        make(nm)
