"""Float64 CPU oracle for fused linear cross-entropy.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code,
constant or helper with the HIP library and is never a fallback for it.

What it computes is the plain textbook definition, in float64, on the exact input
values the GPU receives (bf16 inputs are upcast without rounding):

  targets   y[b, t] = labels[b, t+1] for t < T-1, y[b, T-1] = ignore   (shift)
            y = labels                                                (no shift)
            -- the LoRA-SFT blog post calls ``linear_cross_entropy(hidden,
            weight, labels, ignore_index=-100, shift=True, reduction="mean")``
            with ``labels = input_ids``, so shift means next-token targets
            inside each sequence.
  valid     i is valid iff y_i != ignore_index; n = number of valid rows.
  logits    Z = X . W^T (no bias)  -- ms-swift PR "Add optional fused linear ce
            for qwen2/qwen3 on npu", section "Mathematical Equivalence".
  lse_i     = log sum_v exp(Z_iv)  (computed as m_i + log sum exp(Z_iv - m_i)).
  loss      = sum_valid (lse_i - Z_{i,y_i}) / n   (mean)  or the plain sum;
            reduction "none": the per-row losses l_i = lse_i - Z_{i,y_i}
            (0 on ignored rows), whose negatives are the target log-probs.
  G         = c (softmax(Z_i) - onehot(y_i)) on valid rows, 0 elsewhere,
            c = grad_scale / n (mean) or grad_scale (sum); with "none",
            grad_scale may be a per-row array g (the upstream gradient of the
            per-row losses) and row i uses c_i = g_i.
  grads     dX = G . W and dW = G^T . X, the two identities of the same section.

Three evaluation orders are provided, all meant to agree to rounding:
  * ``global``  -- the whole valid Z at once (small shapes);
  * ``rows``    -- row chunks along the sequence, each chunk doing its own
                   linear + cross-entropy + gradient and summing the weight
                   gradient over chunks, as in the ms-swift PR, section "What
                   this PR does" (chunked autograd in the time dimension);
  * ``vocab``   -- vocabulary slices with an online (max, sum-exp) merge for the
                   forward and d_hidden accumulated slice by slice for the
                   backward, as in Megatron-LM PR "[Dev] Fix Linear-Cross-Entropy
                   Convergence Issue", item 2 (vocabulary split, FP32 d_hidden);
                   the accumulator precision can be simulated ('f64', 'f32',
                   'bf16') to show the effect that PR describes.

Conventions the pages leave open (each is also listed in the design notes):
  * n = 0: loss = 0, dX = dW = 0.          (parity unpinned by the pages)
  * lse of ignored rows is reported as 0.  (parity unpinned by the pages)
  * a valid target outside [0, V) raises ValueError.  (parity unpinned)
  * ignore_index is compared by exact integer equality before the range check.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "targets", "flce", "forward_rows", "dx_rows", "dw_rows", "round_bf16_f64",
]


def _as_f64(a):
    return np.asarray(a, dtype=np.float64)


def targets(labels, shift, ignore_index=-100):
    """Flattened per-row targets y [B*T] (int64) and the validity mask."""
    lab = np.asarray(labels, dtype=np.int64)
    if lab.ndim == 1:
        lab = lab[None, :]
    B, T = lab.shape
    if shift:
        y = np.full((B, T), ignore_index, dtype=np.int64)
        if T > 1:
            y[:, :T - 1] = lab[:, 1:]
    else:
        y = lab.copy()
    y = y.reshape(-1)
    valid = y != ignore_index
    return y, valid


def _check_range(y, valid, V):
    bad = valid & ((y < 0) | (y >= V))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise ValueError(f"target {int(y[i])} of row {i} is outside [0, {V})")


def _scale(reduction, n, grad_scale, N):
    """Gradient factor: a scalar, or for "none" a per-row array [N]."""
    if reduction == "mean":
        return 0.0 if n == 0 else grad_scale / n
    if reduction == "sum":
        return float(grad_scale)
    if reduction == "none":
        return np.broadcast_to(_as_f64(grad_scale), (N,)).copy()
    raise ValueError(f"unknown reduction {reduction!r}")


def _rows_factor(c, rows):
    """c for the given rows, shaped to scale rows of G."""
    return c[rows][:, None] if np.ndim(c) else c


def _row_lse(Z):
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def round_bf16_f64(a):
    """Round float64 values to the nearest-even bfloat16 value (as float64).

    bfloat16 keeps 7 explicit mantissa bits, float64 keeps 52, so the 45 low
    mantissa bits are rounded away (ties to even).  Used only to simulate a BF16
    accumulator for values well inside bf16's exponent range."""
    f = np.ascontiguousarray(a, dtype=np.float64)
    u = f.view(np.uint64)
    drop = np.uint64(52 - 7)
    one = np.uint64(1)
    lsb = (u >> drop) & one
    u = (u + ((one << (drop - one)) - one) + lsb) & ~((one << drop) - one)
    return u.view(np.float64)


def _round_acc(a, acc):
    if acc == "f64":
        return a
    if acc == "f32":
        return a.astype(np.float32).astype(np.float64)
    if acc == "bf16":
        return round_bf16_f64(a)
    raise ValueError(acc)


def flce(X, W, labels, *, ignore_index=-100, reduction="mean", shift=False,
         grad_scale=1.0, mode="global", chunk=None, acc="f64", grads=True):
    """Loss, per-row lse, n_valid and (optionally) dX, dW.

    X: [N, H] (or [B, T, H]); W: [V, H]; labels: [B, T] (or [N] meaning B=1).
    Returns a dict with float64 arrays: loss (scalar), lse [N], n_valid,
    dX [N, H], dW [V, H].
    """
    Xf = _as_f64(X)
    Wf = _as_f64(W)
    if Xf.ndim == 3:
        Xf = Xf.reshape(-1, Xf.shape[-1])
    N, H = Xf.shape
    V = Wf.shape[0]
    y, valid = targets(labels, shift, ignore_index)
    if y.shape[0] != N:
        raise ValueError("labels and hidden states disagree on the row count")
    _check_range(y, valid, V)
    n = int(valid.sum())
    c = _scale(reduction, n, grad_scale, N)
    out = dict(n_valid=n, lse=np.zeros(N), loss=np.zeros(N) if reduction == "none" else 0.0)
    if grads:
        out["dX"] = np.zeros((N, H))
        out["dW"] = np.zeros((V, H))
    if n == 0:
        return out
    if mode == "global":
        _global(Xf, Wf, y, valid, c, reduction, n, out, grads)
    elif mode == "rows":
        _rows(Xf, Wf, y, valid, c, reduction, n, out, grads, chunk or 2048)
    elif mode == "vocab":
        _vocab(Xf, Wf, y, valid, c, reduction, n, out, grads, chunk or 4096, acc)
    else:
        raise ValueError(mode)
    return out


def _finish_loss(out, rows, row_losses, reduction, n):
    """Store the loss: mean or sum of the valid rows' losses, or (none) the
    per-row losses at their rows."""
    if reduction == "none":
        out["loss"][rows] = row_losses
    else:
        s = float(np.sum(row_losses))
        out["loss"] = s / n if reduction == "mean" else s


def _global(X, W, y, valid, c, reduction, n, out, grads):
    rows = np.flatnonzero(valid)
    Xv = X[rows]
    yv = y[rows]
    Z = Xv @ W.T                                   # [n, V]
    lse = _row_lse(Z)
    zt = Z[np.arange(n), yv]
    out["lse"][rows] = lse
    _finish_loss(out, rows, lse - zt, reduction, n)
    if grads:
        P = np.exp(Z - lse[:, None])
        P[np.arange(n), yv] -= 1.0
        G = _rows_factor(c, rows) * P
        out["dX"][rows] = G @ W
        out["dW"][:] = G.T @ Xv


def _rows(X, W, y, valid, c, reduction, n, out, grads, chunk):
    """Chunks along the flattened sequence; each chunk is a small linear +
    cross-entropy whose weight gradient is summed into one buffer."""
    N = X.shape[0]
    all_rows, all_losses = [], []
    for r0 in range(0, N, chunk):
        sl = slice(r0, min(N, r0 + chunk))
        vmask = valid[sl]
        if not vmask.any():
            continue
        rows = r0 + np.flatnonzero(vmask)
        Xc = X[rows]
        yc = y[rows]
        Z = Xc @ W.T
        lse = _row_lse(Z)
        k = np.arange(len(rows))
        all_rows.append(rows)
        all_losses.append(lse - Z[k, yc])
        out["lse"][rows] = lse
        if grads:
            P = np.exp(Z - lse[:, None])
            P[k, yc] -= 1.0
            G = _rows_factor(c, rows) * P
            out["dX"][rows] = G @ W
            out["dW"] += G.T @ Xc
    _finish_loss(out, np.concatenate(all_rows), np.concatenate(all_losses), reduction, n)


def _vocab(X, W, y, valid, c, reduction, n, out, grads, chunk, acc):
    """Vocabulary slices: online max / sum-exp merge, then per-slice gradient
    pieces with d_hidden accumulated slice after slice in precision ``acc``."""
    V = W.shape[0]
    rows = np.flatnonzero(valid)
    Xv = X[rows]
    yv = y[rows]
    m = np.full(n, -np.inf)
    s = np.zeros(n)
    zt = np.zeros(n)
    for v0 in range(0, V, chunk):
        v1 = min(V, v0 + chunk)
        Z = Xv @ W[v0:v1].T
        m_new = np.maximum(m, Z.max(axis=1))
        s = s * np.exp(m - m_new) + np.exp(Z - m_new[:, None]).sum(axis=1)
        m = m_new
        hit = (yv >= v0) & (yv < v1)
        zt[hit] = Z[np.flatnonzero(hit), yv[hit] - v0]
    lse = m + np.log(s)
    out["lse"][rows] = lse
    _finish_loss(out, rows, lse - zt, reduction, n)
    if not grads:
        return
    dX = np.zeros((n, X.shape[1]))
    for v0 in range(0, V, chunk):
        v1 = min(V, v0 + chunk)
        Z = Xv @ W[v0:v1].T
        P = np.exp(Z - lse[:, None])
        hit = np.flatnonzero((yv >= v0) & (yv < v1))
        P[hit, yv[hit] - v0] -= 1.0
        G = _rows_factor(c, rows) * P
        if acc == "f64":
            piece = G @ W[v0:v1]
        else:
            # the slice product is itself formed at FP32 (a GEMM with an FP32
            # accumulator on bf16 operands), only the running sum differs
            piece = (G.astype(np.float32) @ W[v0:v1].astype(np.float32)).astype(np.float64)
        dX = _round_acc(dX + piece, acc)
        out["dW"][v0:v1] = G.T @ Xv
    out["dX"][rows] = dX


# ---------------------------------------------------------------------------
# Row-by-row pieces for large shapes: the same definition evaluated for a few
# chosen rows, so that a sample of a full-size result can be checked exactly.
# ---------------------------------------------------------------------------

def forward_rows(X, W, labels, *, ignore_index=-100, reduction="mean",
                 shift=False, chunk=256, rows=None):
    """lse for every valid row (or only ``rows``), the loss and n_valid.

    Streams over row chunks so that at most [chunk, V] logits exist at once.
    With ``rows`` given, the loss is not computed (it needs every row)."""
    Xf = X  # upcast chunk by chunk to bound memory
    Wf = _as_f64(W)
    N = Xf.shape[0]
    V = Wf.shape[0]
    y, valid = targets(labels, shift, ignore_index)
    _check_range(y, valid, V)
    n = int(valid.sum())
    lse = np.zeros(N)
    want = np.flatnonzero(valid) if rows is None else np.asarray(rows)
    total = 0.0
    for i0 in range(0, len(want), chunk):
        r = want[i0:i0 + chunk]
        Z = _as_f64(Xf[r]) @ Wf.T
        l = _row_lse(Z)
        lse[r] = l
        total += float(np.sum(l - Z[np.arange(len(r)), y[r]]))
    loss = None
    if rows is None:
        loss = 0.0 if n == 0 else (total / n if reduction == "mean" else total)
    return dict(lse=lse, loss=loss, n_valid=n, y=y, valid=valid)


def dx_rows(X, W, y, valid, lse, c, rows):
    """dX[i, :] = sum_v G_iv W_v for the given rows (0 for ignored rows)."""
    Wf = _as_f64(W)
    rows = np.asarray(rows)
    out = np.zeros((len(rows), Wf.shape[1]))
    for k, i in enumerate(rows):
        if not valid[i]:
            continue
        z = _as_f64(X[i]) @ Wf.T
        p = np.exp(z - lse[i])
        p[y[i]] -= 1.0
        out[k] = c * (p @ Wf)
    return out


def dw_rows(X, W, y, valid, lse, c, vocab_ids, chunk=4096):
    """dW[v, :] = sum_i G_iv X_i over valid rows i, for the given vocab ids."""
    vocab_ids = np.asarray(vocab_ids)
    Wv = _as_f64(W[vocab_ids])                   # [k, H]
    rows = np.flatnonzero(valid)
    out = np.zeros((len(vocab_ids), Wv.shape[1]))
    for i0 in range(0, len(rows), chunk):
        r = rows[i0:i0 + chunk]
        Xr = _as_f64(X[r])                        # [c, H]
        P = np.exp(Xr @ Wv.T - lse[r][:, None])   # [c, k]
        P -= (y[r][:, None] == vocab_ids[None, :])
        out += P.T @ Xr
    return c * out


def logits_bytes(N, V, elem_bytes):
    """Size of the [N, V] logits the fused path never allocates."""
    return int(N) * int(V) * int(elem_bytes)


def cosine(a, b):
    """Cosine similarity <a, b> / (|a| |b|) of the two arrays taken as flat
    vectors, in float64: the figure the ms-swift PR, section "Mathematical
    Equivalence", quotes for the chunked gradients against the global ones.
    Convention for zero vectors (the pages fix none): two zero vectors are
    identical (1.0); a zero vector against a nonzero one shares no direction
    (0.0)."""
    a = _as_f64(a).ravel()
    b = _as_f64(b).ravel()
    na = math.sqrt(float(a @ a))
    nb = math.sqrt(float(b @ b))
    if na == 0.0 or nb == 0.0:
        return 1.0 if na == nb else 0.0
    return float(a @ b) / (na * nb)
