"""Pins for the float64 oracle: each test checks it against something other than
itself -- a hand-worked example, a closed form, a textbook special case, brute
force, finite differences or an algebraic invariant -- so that a dropped term,
a wrong sign or index, a wrong denominator or a transposed operand fails one.
CPU only."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _problem(seed, B=2, T=9, H=6, V=11, ignore_frac=0.3, w_std=0.5):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((B * T, H))
    W = w_std * rng.standard_normal((V, H))
    lab = rng.integers(0, V, size=(B, T))
    lab[rng.random((B, T)) < ignore_frac] = -100
    return X, W, lab


# --- hand-worked example (golden fixture) --------------------------------

def test_hand_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "hand_worked_3x2x3.json")))
    X = np.array(ex["X"])
    W = np.array(ex["W"])
    for case in ex["cases"]:
        for mode in ("global", "rows", "vocab"):
            r = oracle.flce(X, W, np.array(case["labels"]), shift=case["shift"],
                            reduction=case["reduction"], mode=mode, chunk=2)
            assert r["n_valid"] == case["n_valid"]
            assert r["loss"] == pytest.approx(case["loss"], rel=1e-14, abs=1e-14)
            np.testing.assert_allclose(r["lse"], case["lse"], rtol=1e-14, atol=1e-14)
            np.testing.assert_allclose(r["dX"], case["dX"], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(r["dW"], case["dW"], rtol=1e-13, atol=1e-15)


def test_pages_memory_figure():
    f = json.load(open(os.path.join(GOLDEN, "pages_memory_figure.json")))
    N = f["B"] * f["Seq"]
    two_bf16 = 2 * oracle.logits_bytes(N, f["vocab"], 2)
    assert two_bf16 > f["logits_plus_grad_more_than_bytes"]
    assert oracle.logits_bytes(N, f["vocab"], 4) == two_bf16
    assert two_bf16 < 1.2 * f["logits_plus_grad_more_than_bytes"]


# --- C1: chunked == global (exact in real arithmetic) ----------------------

@pytest.mark.parametrize("reduction", ["mean", "sum"])
@pytest.mark.parametrize("shift", [False, True])
def test_chunked_equals_global(reduction, shift):
    X, W, lab = _problem(1, B=3, T=17, H=8, V=29)
    g = oracle.flce(X, W, lab, reduction=reduction, shift=shift, grad_scale=0.7)
    runs = [("rows", c) for c in (1, 7, 2048, X.shape[0])] + \
           [("vocab", c) for c in (1, 3, 10, 29, 4096)]
    for mode, c in runs:
        r = oracle.flce(X, W, lab, reduction=reduction, shift=shift,
                        grad_scale=0.7, mode=mode, chunk=c)
        assert r["n_valid"] == g["n_valid"]
        assert r["loss"] == pytest.approx(g["loss"], rel=1e-12)
        np.testing.assert_allclose(r["lse"], g["lse"], rtol=1e-12, atol=1e-13)
        for k in ("dX", "dW"):
            np.testing.assert_allclose(r[k], g[k], rtol=1e-11, atol=1e-14)
            assert f"{oracle.cosine(r[k], g[k]):.6f}" == "1.000000"


# --- C2: W = 0 --------------------------------------------------------------

@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_zero_weight_closed_form(reduction):
    X, W, lab = _problem(2, V=13)
    W[:] = 0.0
    V = W.shape[0]
    r = oracle.flce(X, W, lab, reduction=reduction)
    y, valid = oracle.targets(lab, False)
    n = int(valid.sum())
    expect_loss = math.log(V) if reduction == "mean" else n * math.log(V)
    assert r["loss"] == pytest.approx(expect_loss, rel=1e-14)
    np.testing.assert_allclose(r["lse"][valid], math.log(V), rtol=1e-15)
    assert np.all(r["lse"][~valid] == 0.0)
    assert np.all(r["dX"] == 0.0)
    c = 1.0 / n if reduction == "mean" else 1.0
    xs = X[valid].sum(axis=0)
    expect = np.empty_like(r["dW"])
    for v in range(V):
        expect[v] = c * (xs / V - X[valid & (y == v)].sum(axis=0))
    np.testing.assert_allclose(r["dW"], expect, rtol=1e-12, atol=1e-14)


# --- C3: X = 0 --------------------------------------------------------------

def test_zero_hidden_closed_form():
    X, W, lab = _problem(3, V=7)
    X[:] = 0.0
    r = oracle.flce(X, W, lab, shift=True)
    y, valid = oracle.targets(lab, True)
    n = int(valid.sum())
    assert r["loss"] == pytest.approx(math.log(W.shape[0]), rel=1e-14)
    assert np.all(r["dW"] == 0.0)
    wbar = W.mean(axis=0)
    for i in range(X.shape[0]):
        want = (wbar - W[y[i]]) / n if valid[i] else np.zeros(W.shape[1])
        np.testing.assert_allclose(r["dX"][i], want, rtol=1e-12, atol=1e-15)


# --- C4: rows of G sum to zero ----------------------------------------------

def test_weight_grad_columns_sum_to_zero():
    X, W, lab = _problem(4, V=31)
    r = oracle.flce(X, W, lab, reduction="sum")
    scale = np.abs(r["dW"]).max()
    assert np.abs(r["dW"].sum(axis=0)).max() < 1e-13 * scale * W.shape[0]


# --- C5: ignored rows contribute nothing ------------------------------------

@pytest.mark.parametrize("mode", ["global", "rows", "vocab"])
def test_ignored_rows_are_never_read(mode):
    X, W, lab = _problem(5, B=2, T=12, H=5, V=9)
    for shift in (False, True):
        y, valid = oracle.targets(lab, shift)
        a = oracle.flce(X, W, lab, shift=shift, mode=mode, chunk=4)
        X2 = X.copy()
        X2[~valid] = 1e6 * np.random.default_rng(0).standard_normal(X2[~valid].shape)
        b = oracle.flce(X2, W, lab, shift=shift, mode=mode, chunk=4)
        assert a["loss"] == b["loss"]
        assert np.array_equal(a["lse"], b["lse"])
        assert np.array_equal(a["dW"], b["dW"])
        assert np.array_equal(a["dX"], b["dX"])
        assert np.all(b["dX"][~valid] == 0.0)


# --- C6: finite differences -------------------------------------------------

@pytest.mark.parametrize("shift", [False, True])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_finite_differences(shift, reduction):
    X, W, lab = _problem(6, B=2, T=3, H=4, V=5, ignore_frac=0.2)
    lab[0, 1] = -100
    gs = 1.3
    r = oracle.flce(X, W, lab, shift=shift, reduction=reduction, grad_scale=gs)

    def loss(Xa, Wa):
        return gs * oracle.flce(Xa, Wa, lab, shift=shift, reduction=reduction,
                                grads=False)["loss"]

    h = 1e-6
    for name, A, G in (("X", X, r["dX"]), ("W", W, r["dW"])):
        num = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            Ap = A.copy()
            Am = A.copy()
            Ap[idx] += h
            Am[idx] -= h
            if name == "X":
                num[idx] = (loss(Ap, W) - loss(Am, W)) / (2 * h)
            else:
                num[idx] = (loss(X, Ap) - loss(X, Am)) / (2 * h)
        scale = np.abs(num).max()
        assert np.abs(num - G).max() <= 1e-7 * scale, name


# --- C7: V = 2 is logistic regression ---------------------------------------

def test_two_classes_is_logistic():
    X, W, lab = _problem(7, V=2, ignore_frac=0.0)
    r = oracle.flce(X, W, lab, reduction="sum")
    y, _ = oracle.targets(lab, False)
    Z = X @ W.T
    total = 0.0
    for i in range(X.shape[0]):
        d = Z[i, 1 - y[i]] - Z[i, y[i]]
        total += math.log1p(math.exp(d)) if d < 30 else d + math.log1p(math.exp(-d))
    assert r["loss"] == pytest.approx(total, rel=1e-13)


# --- C8: brute force with exactly-rounded sums ------------------------------

def test_bruteforce_rowwise():
    X, W, lab = _problem(8, B=1, T=6, H=3, V=7)
    r = oracle.flce(X, W, lab)
    y, valid = oracle.targets(lab, False)
    losses = []
    for i in range(X.shape[0]):
        if not valid[i]:
            continue
        z = [math.fsum(X[i, h] * W[v, h] for h in range(X.shape[1]))
             for v in range(W.shape[0])]
        lse = math.log(math.fsum(math.exp(t) for t in z))
        assert r["lse"][i] == pytest.approx(lse, rel=1e-14, abs=1e-14)
        losses.append(lse - z[y[i]])
    assert r["loss"] == pytest.approx(math.fsum(losses) / len(losses), rel=1e-14)


# --- C9: shift = next-token targets inside each sequence ---------------------

def test_shift_equals_manual_realignment():
    B, T, H, V = 3, 10, 5, 8
    rng = np.random.default_rng(9)
    X = rng.standard_normal((B, T, H))
    W = rng.standard_normal((V, H))
    lab = rng.integers(0, V, size=(B, T))
    lab[1, :4] = -100
    a = oracle.flce(X.reshape(-1, H), W, lab, shift=True)
    b = oracle.flce(X[:, :T - 1].reshape(-1, H), W, lab[:, 1:], shift=False)
    assert a["n_valid"] == b["n_valid"] == B * (T - 1) - 3
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-14)
    dXa = a["dX"].reshape(B, T, H)
    np.testing.assert_allclose(dXa[:, :T - 1].reshape(-1, H), b["dX"], rtol=1e-13, atol=1e-16)
    assert np.all(dXa[:, T - 1] == 0.0)
    np.testing.assert_allclose(a["dW"], b["dW"], rtol=1e-12, atol=1e-16)


# --- C10: reductions and grad_scale ----------------------------------------

def test_reduction_and_grad_scale_relations():
    X, W, lab = _problem(10)
    m = oracle.flce(X, W, lab, reduction="mean")
    s = oracle.flce(X, W, lab, reduction="sum")
    s3 = oracle.flce(X, W, lab, reduction="sum", grad_scale=-3.0)
    n = m["n_valid"]
    assert s["loss"] == pytest.approx(n * m["loss"], rel=1e-14)
    np.testing.assert_allclose(s["dX"] / n, m["dX"], rtol=1e-13, atol=1e-17)
    np.testing.assert_allclose(s["dW"] / n, m["dW"], rtol=1e-13, atol=1e-17)
    np.testing.assert_allclose(s3["dW"], -3.0 * s["dW"], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(s3["dX"], -3.0 * s["dX"], rtol=1e-13, atol=1e-16)


# --- C11: permutations -------------------------------------------------------

def test_row_and_vocab_permutations():
    X, W, lab = _problem(11, B=1, T=20, V=10)
    r = oracle.flce(X, W, lab, reduction="sum")
    rng = np.random.default_rng(11)
    p = rng.permutation(X.shape[0])
    rp = oracle.flce(X[p], W, lab[:, p], reduction="sum")
    assert rp["loss"] == pytest.approx(r["loss"], rel=1e-13)
    np.testing.assert_allclose(rp["lse"], r["lse"][p], rtol=1e-14)
    np.testing.assert_allclose(rp["dX"], r["dX"][p], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(rp["dW"], r["dW"], rtol=1e-12, atol=1e-15)
    q = rng.permutation(W.shape[0])          # new id k holds old id q[k]
    inv = np.argsort(q)
    lab2 = np.where(lab == -100, -100, inv[np.where(lab == -100, 0, lab)])
    rq = oracle.flce(X, W[q], lab2, reduction="sum")
    assert rq["loss"] == pytest.approx(r["loss"], rel=1e-13)
    np.testing.assert_allclose(rq["dW"], r["dW"][q], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(rq["dX"], r["dX"], rtol=1e-12, atol=1e-16)


# --- C12: a common shift of every weight row --------------------------------

def test_common_weight_shift_invariance():
    X, W, lab = _problem(12)
    a = np.random.default_rng(12).standard_normal(W.shape[1])
    r = oracle.flce(X, W, lab)
    r2 = oracle.flce(X, W + a[None, :], lab)
    _, valid = oracle.targets(lab, False)
    assert r2["loss"] == pytest.approx(r["loss"], rel=1e-12)
    np.testing.assert_allclose(r2["dX"], r["dX"], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(r2["dW"], r["dW"], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(r2["lse"][valid], r["lse"][valid] + X[valid] @ a,
                               rtol=1e-12)


# --- C13: counting under shift for the full-size masks ----------------------

@pytest.mark.parametrize("B,T,prefix,n", [(1, 8192, 1638, 6554), (1, 32768, 8192, 24576)])
def test_valid_count_under_shift_with_prefix_mask(B, T, prefix, n):
    lab = np.arange(B * T, dtype=np.int64).reshape(B, T) % 1000
    lab[:, :prefix] = -100
    y, valid = oracle.targets(lab, True)
    assert int(valid.sum()) == n
    assert not valid.reshape(B, T)[:, -1].any()


# --- C14: BF16 vs FP32 accumulation of d_hidden over vocabulary slices ------

def test_bf16_accumulation_is_measurably_worse():
    rng = np.random.default_rng(14)
    N, H, V = 24, 32, 4000
    X = rng.standard_normal((N, H))
    W = 0.05 * rng.standard_normal((V, H))
    lab = rng.integers(0, V, size=(1, N))
    exact = oracle.flce(X, W, lab, mode="vocab", chunk=100)["dX"]
    f32 = oracle.flce(X, W, lab, mode="vocab", chunk=100, acc="f32")["dX"]
    b16 = oracle.flce(X, W, lab, mode="vocab", chunk=100, acc="bf16")["dX"]
    e32 = np.abs(f32 - exact).max()
    e16 = np.abs(b16 - exact).max()
    assert e16 > 50 * e32
    assert oracle.cosine(f32, exact) > 0.99999999


def test_bf16_rounding_helper():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -12,
                     -2.5 - 2 ** -7, 3.0e-20])
    got = oracle.round_bf16_f64(vals)
    want = [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, None]  # ties go to even
    for g, w, v in zip(got, want, vals):
        if w is None:
            assert abs(g - v) <= abs(v) * 2 ** -8
        else:
            assert g == w, (v, g, w)


# --- conventions the pages leave open (parity unpinned) ---------------------

def test_no_valid_rows_convention():
    X, W, lab = _problem(15)
    lab[:] = -100
    r = oracle.flce(X, W, lab)
    assert r["n_valid"] == 0 and r["loss"] == 0.0
    assert not r["dX"].any() and not r["dW"].any() and not r["lse"].any()


def test_out_of_range_label_raises():
    X, W, lab = _problem(16, V=5)
    lab[0, 0] = 5
    with pytest.raises(ValueError):
        oracle.flce(X, W, lab)
    lab[0, 0] = -1
    with pytest.raises(ValueError):
        oracle.flce(X, W, lab)


def test_ignore_index_inside_vocab_range():
    X, W, lab = _problem(17, V=6, ignore_frac=0.0)
    lab[0, :3] = 2
    r = oracle.flce(X, W, lab, ignore_index=2)
    y, valid = oracle.targets(lab, False, ignore_index=2)
    assert r["n_valid"] == int((lab != 2).sum())
    assert np.all(r["dX"][~valid] == 0.0)


# --- the row-by-row helpers used for full-size samples ----------------------

def test_row_helpers_match_full_oracle():
    X, W, lab = _problem(18, B=2, T=40, H=7, V=23)
    for reduction in ("mean", "sum"):
        for shift in (False, True):
            r = oracle.flce(X, W, lab, reduction=reduction, shift=shift, grad_scale=0.5)
            f = oracle.forward_rows(X, W, lab, reduction=reduction, shift=shift, chunk=7)
            assert f["n_valid"] == r["n_valid"]
            assert f["loss"] == pytest.approx(r["loss"], rel=1e-13)
            np.testing.assert_allclose(f["lse"], r["lse"], rtol=1e-14)
            n = f["n_valid"]
            c = 0.5 / n if reduction == "mean" else 0.5
            rows = [0, 5, 39, 79]
            np.testing.assert_allclose(
                oracle.dx_rows(X, W, f["y"], f["valid"], f["lse"], c, rows),
                r["dX"][rows], rtol=1e-12, atol=1e-16)
            vids = [0, 3, 22]
            np.testing.assert_allclose(
                oracle.dw_rows(X, W, f["y"], f["valid"], f["lse"], c, vids, chunk=9),
                r["dW"][vids], rtol=1e-12, atol=1e-16)


# --- C15: reduction "none" (per-token losses, per-token upstream gradients) --

@pytest.mark.parametrize("mode", ["global", "rows", "vocab"])
def test_per_row_losses_are_negative_log_softmax(mode):
    """Each valid row's loss is -log_softmax(z_i)[y_i] (scipy's routine on the
    textbook logits), 0 on ignored rows; the target log-prob is its negative."""
    from scipy.special import log_softmax
    X, W, lab = _problem(15, B=2, T=7, H=5, V=13)
    r = oracle.flce(X, W, lab, shift=True, reduction="none", mode=mode, chunk=3)
    y, valid = oracle.targets(lab, True)
    ls = log_softmax(X @ W.T, axis=1)
    want = np.where(valid, -ls[np.arange(len(y)), np.where(valid, y, 0)], 0.0)
    np.testing.assert_allclose(r["loss"], want, rtol=1e-13, atol=1e-13)
    s = oracle.flce(X, W, lab, shift=True, reduction="sum", grads=False)
    assert float(np.sum(r["loss"])) == pytest.approx(s["loss"], rel=1e-13)


@pytest.mark.parametrize("mode", ["global", "rows", "vocab"])
def test_per_row_upstream_gradient_finite_differences(mode):
    """With reduction "none" and per-row weights g, dX and dW are the
    gradients of sum_i g_i l_i (central finite differences)."""
    X, W, lab = _problem(16, B=2, T=3, H=4, V=5, ignore_frac=0.2)
    g = np.random.default_rng(0).standard_normal(X.shape[0])
    r = oracle.flce(X, W, lab, reduction="none", grad_scale=g, mode=mode, chunk=2)

    def loss(Xa, Wa):
        return float(g @ oracle.flce(Xa, Wa, lab, reduction="none", grads=False)["loss"])

    h = 1e-6
    for name, A, G in (("X", X, r["dX"]), ("W", W, r["dW"])):
        num = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            Ap = A.copy()
            Am = A.copy()
            Ap[idx] += h
            Am[idx] -= h
            if name == "X":
                num[idx] = (loss(Ap, W) - loss(Am, W)) / (2 * h)
            else:
                num[idx] = (loss(X, Ap) - loss(X, Am)) / (2 * h)
        assert np.abs(num - G).max() <= 1e-7 * np.abs(num).max(), name


def test_uniform_per_row_weights_equal_mean():
    X, W, lab = _problem(17, B=2, T=8, H=6, V=9)
    m = oracle.flce(X, W, lab, reduction="mean", grad_scale=0.8)
    n = m["n_valid"]
    r = oracle.flce(X, W, lab, reduction="none", grad_scale=np.full(X.shape[0], 0.8 / n))
    np.testing.assert_allclose(r["dX"], m["dX"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["dW"], m["dW"], rtol=1e-12, atol=1e-15)


# --- the cosine metric every gradient-parity check uses ------------------

def test_cosine_hand_values():
    """oracle.cosine against values fixed by plane geometry, not by its own
    formula: orthogonal, antiparallel and 45-degree vectors, invariance under
    positive scaling and under reshaping, sign under negation, an asymmetric
    pair (a formula that divided by |a|^2 would fail it), and the zero-vector
    convention."""
    assert oracle.cosine([1.0, 0.0], [0.0, 1.0]) == 0.0
    assert oracle.cosine([1.0, 0.0], [-3.0, 0.0]) == pytest.approx(-1.0, abs=1e-15)
    assert oracle.cosine([1.0, 0.0], [1.0, 1.0]) == pytest.approx(1.0 / math.sqrt(2.0),
                                                                  rel=1e-15)
    # 3-4-5 and 5-12-13 right triangles: cos = (3*5 + 4*12) / (5 * 13) = 63/65
    assert oracle.cosine([3.0, 4.0], [5.0, 12.0]) == pytest.approx(63.0 / 65.0, rel=1e-15)
    assert oracle.cosine([3.0, 4.0], [50.0, 120.0]) == pytest.approx(63.0 / 65.0, rel=1e-15)
    assert oracle.cosine([-3.0, -4.0], [5.0, 12.0]) == pytest.approx(-63.0 / 65.0, rel=1e-15)
    # the arrays are compared as flat vectors, whatever their shape
    a = np.array([[3.0, 0.0], [0.0, 4.0]])
    b = np.array([[5.0, 0.0], [0.0, 12.0]])
    assert oracle.cosine(a, b) == pytest.approx(63.0 / 65.0, rel=1e-15)
    # nearly parallel vectors: 1 - cos = 1 - 1/sqrt(1 + e^2) ~ e^2 / 2, resolved
    e = 1e-4
    assert 1.0 - oracle.cosine([1.0, 0.0], [1.0, e]) == pytest.approx(e * e / 2, rel=1e-6)
    # zero vectors: identical when both are zero, no direction shared otherwise
    assert oracle.cosine([0.0, 0.0], [0.0, 0.0]) == 1.0
    assert oracle.cosine([0.0, 0.0], [1.0, 2.0]) == 0.0
    assert oracle.cosine([1.0, 2.0], [0.0, 0.0]) == 0.0


def test_cosine_detects_a_wrong_softmax_part():
    """The gradient checks rest on the cosine telling a correct gradient from
    one whose softmax part is missing: with the softmax term dropped the dW
    cosine falls measurably (here below 0.9999999), and a gradient with the
    opposite sign gives -1."""
    X, W, lab = _problem(21, B=2, T=40, H=8, V=30, w_std=1.0)
    r = oracle.flce(X, W, lab)
    y, valid = oracle.targets(lab, False, -100)
    onehot_only = np.zeros_like(r["dW"])
    c = 1.0 / r["n_valid"]
    for i in np.flatnonzero(valid):
        onehot_only[y[i]] -= c * X[i]
    assert oracle.cosine(r["dW"], onehot_only) < 0.9999999
    assert oracle.cosine(r["dW"], -r["dW"]) == pytest.approx(-1.0, abs=1e-15)
    assert oracle.cosine(r["dW"], 3.0 * r["dW"]) == pytest.approx(1.0, abs=1e-15)
