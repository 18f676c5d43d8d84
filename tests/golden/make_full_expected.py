"""Write the float64 oracle's expected values for the four full-size bf16
workloads (and the full tiny fp32 one) to tests/golden/full_<name>.npz.

Only ``synth`` (inputs) and ``oracle`` (arithmetic) are used.  Stored per
workload: n_valid, the loss, lse of every row, and dX / dW on sampled rows
(float32: the tests' tolerances are far above its rounding):
  * dX rows: the first and last valid rows, an ignored row, random rows, and
    the rows on both sides of every 256-row tile edge of the compacted valid
    rows (compacted indices 256 k - 1 and 256 k, mapped back to their rows);
  * dW rows: the most frequent targets, a target-free id, the last vocabulary
    rows (the ragged last tile), random ids, and the first and last column of
    every vocabulary block the backward works in (block_widths below).

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


def block_widths(N, H, V, es):
    """Vocabulary block widths of the backward at this shape: the recompute
    path's (two softmax-gradient slabs within 512 MiB for the padded rows, or
    within 1 GiB to come closer to 8192 columns; W rows of a block and the
    slab below 2^31 bytes; a multiple of 256) and
    the chunked mode's (32768, or narrower so that a block's W rows stay below
    2^31 bytes).  They only place samples: a change of the library's blocking
    moves the edges away from the samples, it does not make a sample wrong."""
    rows_pad = -(-N // 256) * 256
    per_col = 2 * rows_pad * es
    vb = max((512 << 20) // per_col, min(8192, (1024 << 20) // per_col))
    vb = min(vb, 0x7FFFFFFF // (rows_pad * es), 0x7FFFFFFF // (H * es))
    vb = max(256, vb // 256 * 256)
    vb = min(vb, -(-V // 256) * 256)
    cb = max(256, min(32768, 0x7FFFFFFF // (H * es)) // 256 * 256)
    return vb, cb


def sample_rows(y, valid, seed):
    rng = np.random.default_rng(seed)
    vrows = np.flatnonzero(valid)
    pick = {int(vrows[0]), int(vrows[-1])}
    for k in range(256, len(vrows), 256):   # token-tile edges of the valid rows
        pick.update({int(vrows[k - 1]), int(vrows[k])})
    ign = np.flatnonzero(~valid)
    if len(ign):
        pick.add(int(ign[len(ign) // 2]))
    while len(pick) < N_DX:
        pick.add(int(rng.choice(vrows)))
    return np.array(sorted(pick))


def sample_vocab(y, valid, V, seed, widths):
    rng = np.random.default_rng(seed)
    counts = np.bincount(y[valid], minlength=V)
    top = np.argsort(-counts, kind="stable")[:4]
    pick = {int(t) for t in top}
    for wdt in widths:                        # both edges of every block
        for b0 in range(0, V, wdt):
            pick.update({b0, min(b0 + wdt, V) - 1})
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
    es = 2 if w.dtype == "bf16" else 4
    widths = block_widths(w.N, w.H, w.V, es)
    vids = sample_vocab(f["y"], f["valid"], w.V, 8, widths)
    dx = oracle.dx_rows(w.X, w.W, f["y"], f["valid"], f["lse"], c, rows)
    dw = oracle.dw_rows(w.X, w.W, f["y"], f["valid"], f["lse"], c, vids)
    out = os.path.join(HERE, f"full_{name}.npz")
    np.savez_compressed(out, n_valid=n, loss=f["loss"], lse=f["lse"],
                        dx_rows=rows, dx=dx.astype(np.float32), dw_rows=vids,
                        dw=dw.astype(np.float32), grad_scale=1.0,
                        block_widths=np.array(widths))
    print(f"{name}: {len(rows)} dX rows, {len(vids)} dW rows, blocks {widths}", flush=True)
    print(f"{name}: n={n} loss={f['loss']:.10f} ({time.time() - t0:.1f}s) -> {out}",
          flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or list(synth.WORKLOADS)
    for nm in names:
        make(nm)
