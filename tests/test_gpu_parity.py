"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Oracle-sized cases keep each workload's recipe (distributions, masks, shift,
reduction, dtype) at sizes that span several 256-wide tiles in both N and V and
end in ragged tails; the full-size workloads are checked on the oracle's stored
values (tests/golden/full_*.npz: loss, every row's lse, sampled dX and dW rows)
and on invariants that hold at any size."""
import os

import numpy as np
import pytest
import torch

import lm_head_linear_flce_amd as F
import oracle
import synth
from gpu_util import (DEV, check, check_block_coverage, check_sampled_rows, run,
                      run_chunked, soft_parts, soft_tolerance, to_device)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# (workload recipe, overrides): several tiles in N and V, ragged tails
SMALL = [
    ("tiny_f32", {}),
    ("tiny_f32", dict(B=3, T=211, H=104, V=1000, seed=11)),
    ("qwen2_7b_head", dict(T=777, H=512, V=3001, seed=21)),
    ("qwen3_sft_batch", dict(T=613, H=392, V=5003, seed=31)),
    ("long_context", dict(T=2049, H=256, V=2051, seed=41)),
    ("ragged_vocab", dict(T=1031, H=128, V=4099, seed=51)),
    # N large enough that the backward splits the vocabulary into blocks
    ("qwen2_7b_head", dict(T=8193, H=64, V=40013, seed=61)),
    # forward work items of several vocabulary tiles (the later ones start
    # from LDS stages filled during the previous tile's epilogue) with H
    # ending in a partial K step (bf16: 400 of 512 bytes; fp32: 800 of 896)
    ("qwen2_7b_head", dict(T=6600, H=200, V=20011, seed=71)),
    ("tiny_f32", dict(B=2, T=3300, H=200, V=20011, seed=72)),
]


def _ids(p):
    name, ov = p
    return name + ("" if not ov else "-" + "-".join(f"{k}{v}" for k, v in ov.items()
                                                    if k != "seed"))


@pytest.mark.parametrize("case", SMALL, ids=[_ids(p) for p in SMALL])
def test_small_parity(case):
    name, ov = case
    w = synth.workload(name, **ov)
    print(f"[parity] {name} {ov} N={w.N} H={w.H} V={w.V}", flush=True)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="rows", chunk=1024)
    got = run(w)
    check(w, got, ref, what=name)
    # ignored rows of dX are exactly zero
    _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    assert np.all(got["dX"][~valid] == 0.0)


@pytest.mark.parametrize("case", SMALL[2:4], ids=[_ids(p) for p in SMALL[2:4]])
def test_fp32_gradient_outputs(case):
    """grad_dtype=float32 returns the FP32 accumulators unrounded."""
    name, ov = case
    w = synth.workload(name, **ov)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="rows", chunk=1024)
    got = run(w, grad_dtype=torch.float32)
    cos = check(w, got, ref, what=name)
    assert cos["dX"] > 0.99999 and cos["dW"] > 0.99999


@pytest.mark.parametrize("case", SMALL[:5], ids=[_ids(p) for p in SMALL[:5]])
def test_softmax_part_of_the_gradients(case):
    """The contract's tolerances are dominated by the one-hot term (the
    softmax is diffuse at these shapes), so the softmax part alone is compared
    too, with the FP32 gradient outputs: its direction (cosine) and its size
    (norm ratio), for both gradients."""
    name, ov = case
    w = synth.workload(name, **ov)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="rows", chunk=1024)
    got = run(w, grad_dtype=torch.float32)
    n = ref["n_valid"]
    gx, gw = soft_parts(w, got["dX"], got["dW"], n)
    rx, rw = soft_parts(w, ref["dX"], ref["dW"], n)
    cx, cw = oracle.cosine(gx, rx), oracle.cosine(gw, rw)
    print(f"[soft part] {name}: cos P.W {cx:.7f}  cos P^T.X {cw:.7f}", flush=True)
    rnx = np.linalg.norm(gx) / np.linalg.norm(rx)
    rnw = np.linalg.norm(gw) / np.linalg.norm(rw)
    # fp32 G: the soft parts to rounding; bf16 G: see soft_tolerance
    cmin, rtol = soft_tolerance(w)
    assert cx >= cmin and cw >= cmin, (cx, cw)
    assert abs(rnx - 1) <= rtol and abs(rnw - 1) <= rtol, (rnx, rnw)


def test_grad_scale_and_autograd():
    w = synth.workload("qwen2_7b_head", T=300, H=128, V=700, seed=71)
    X, W, lab = to_device(w)
    Xr = X.detach().clone().requires_grad_(True)
    Wr = W.detach().clone().requires_grad_(True)
    loss = F.linear_cross_entropy(Xr, Wr, lab, ignore_index=-100, shift=True,
                                  reduction="mean")
    (2.5 * loss).backward()
    ref = oracle.flce(w.X, w.W, w.labels, shift=True, grad_scale=2.5)
    assert abs(float(loss.detach()) - ref["loss"]) <= 2e-3 * abs(ref["loss"])
    gx = Xr.grad.reshape(w.N, w.H).double().cpu().numpy()
    gw = Wr.grad.double().cpu().numpy()
    assert oracle.cosine(gx, ref["dX"]) >= 0.9999
    assert oracle.cosine(gw, ref["dW"]) >= 0.9999
    assert np.abs(gx - ref["dX"]).max() <= 1e-2 * np.abs(ref["dX"]).max()
    assert np.abs(gw - ref["dW"]).max() <= 1e-2 * np.abs(ref["dW"]).max()


def test_outputs_are_bitwise_deterministic():
    # fixed reduction orders everywhere: loss, lse, dX (read-modify-write by a
    # single owner per launch, launches in stream order) and dW
    w = synth.workload("ragged_vocab", T=900, H=256, V=3001, seed=81)
    X, W, lab = to_device(w)
    outs = []
    for _ in range(3):
        loss, lse, _, _ = F.forward(X, W, lab, -100, w.shift, w.reduction)
        dX, dW, _ = F.backward(X, W, lab, lse, shift=w.shift, reduction=w.reduction)
        outs.append((loss, lse, dX, dW))
    torch.cuda.synchronize()
    assert len({float(o[0]) for o in outs}) == 1
    for o in outs[1:]:
        for k in (1, 2, 3):
            assert torch.equal(o[k], outs[0][k])


def test_ignored_rows_are_never_read():
    w = synth.workload("qwen3_sft_batch", T=300, H=128, V=1000, seed=91)
    _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    a = run(w)
    w2 = synth.workload("qwen3_sft_batch", T=300, H=128, V=1000, seed=91)
    ign = np.flatnonzero(~valid)
    noise = np.random.default_rng(0).standard_normal((len(ign), w.H)) * 1e4
    w2.X[ign] = synth.round_to_bf16(noise.astype(np.float32))
    w2.X[ign[:3]] = np.nan
    b = run(w2)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["lse"], b["lse"])
    assert np.array_equal(a["dW"], b["dW"])
    assert np.all(b["dX"][~valid] == 0.0)
    assert np.array_equal(b["dX"][valid], a["dX"][valid])


def test_no_valid_rows():
    w = synth.workload("long_context", T=500, H=64, V=300, seed=101)
    w.labels[:] = -100
    got = run(w)
    assert got["n_valid"] == 0 and got["loss"] == 0.0
    assert not got["dX"].any() and not got["dW"].any() and not got["lse"].any()


def test_single_token_sequences_with_shift():
    w = synth.workload("qwen2_7b_head", B=5, T=1, H=64, V=300, seed=111)
    got = run(w)
    assert got["n_valid"] == 0 and got["loss"] == 0.0


def test_empty_batch():
    X = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    W = torch.randn((300, 64), device=DEV).to(torch.bfloat16)
    lab = torch.zeros((0, 0), dtype=torch.int64, device=DEV).reshape(1, 0)
    loss, lse, n, st = F.forward(X, W, lab)
    torch.cuda.synchronize()
    assert float(loss) == 0.0 and int(n) == 0 and int(st) == 0


def test_label_out_of_range_sets_status_and_nan():
    w = synth.workload("ragged_vocab", T=300, H=64, V=500, seed=121)
    w.labels[0, 5] = w.V + 3
    got = run(w)
    assert got["status"] == F.FLCE_ERR_LABEL_RANGE
    assert got["bstatus"] == F.FLCE_ERR_LABEL_RANGE
    assert np.isnan(got["loss"])
    assert np.isnan(got["dW"]).any()


def test_ignore_index_inside_vocabulary():
    w = synth.workload("ragged_vocab", T=400, H=64, V=600, seed=131)
    w.labels[w.labels < 50] = 7
    w.ignore_index = 7
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=7, reduction=w.reduction)
    got = run(w)
    check(w, got, ref, what="ignore=7")


def test_zero_weight_gives_log_vocab():
    w = synth.workload("qwen2_7b_head", T=500, H=128, V=1500, seed=141)
    w.W[:] = 0.0
    got = run(w)
    assert abs(got["loss"] - np.log(w.V)) <= 1e-5 * np.log(w.V)
    _, valid = oracle.targets(w.labels, w.shift)
    assert np.abs(got["lse"][valid] - np.log(w.V)).max() < 1e-5
    assert not got["dX"].any()


def test_peak_memory_never_holds_logits():
    # the device memory a call takes beyond its inputs is the caller's
    # workspace plus the outputs; the workspace is linear in N and grows with
    # V only by the 4-byte vocabulary-to-one-hot-row map (the gradient slabs
    # are a fixed budget); at this shape the logits would be 4.3 GB
    w = synth.workload("long_context", T=8192, H=128, V=262144, seed=151)
    ws_v = [F.flce_workspace_size(w.B, w.T, w.H, v, F.FLCE_DTYPE_BF16) for v in (w.V, 4 * w.V)]
    assert 0 <= ws_v[1] - ws_v[0] <= 4 * (3 * w.V) + 256, ws_v
    X, W, lab = to_device(w)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    loss, lse, _, _ = F.forward(X, W, lab, -100, w.shift, w.reduction)
    dX, dW, _ = F.backward(X, W, lab, lse, shift=w.shift, reduction=w.reduction)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    ws = F.flce_workspace_size(w.B, w.T, w.H, w.V, F.FLCE_DTYPE_BF16)
    outs = (w.N * w.H + w.V * w.H) * 2 + w.N * 4 + 4096
    assert peak <= ws + outs + (2 << 20), (peak, ws, outs)
    assert peak < w.N * w.V * 2 / 4


@pytest.mark.parametrize("dtype,V", [("bf16", 16640), ("f32", 8448)])
def test_widest_hidden_size(dtype, V):
    """H = 65536, the widest the ABI takes.  A block of W rows then reaches the
    2^31 bytes one buffer descriptor addresses, so both modes narrow their
    vocabulary blocks (two blocks here, the second one ragged); loss, lse and
    dX in full and sampled dW rows against the oracle."""
    w = synth.workload("tiny_f32", B=1, T=8, H=65536, V=V, dtype=dtype, seed=171, mask_arg=2)
    print(f"[widest] N={w.N} H={w.H} V={w.V} {dtype}", flush=True)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="rows", chunk=8)
    y, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([y[valid], rng.integers(0, w.V, 48), [w.V - 1]]))
    X, W, lab = to_device(w)
    for mode in ("recompute", "chunked"):
        if mode == "recompute":
            loss, lse, n_valid, status = F.forward(X, W, lab, w.ignore_index, w.shift,
                                                   w.reduction)
            dX, dW, bstatus = F.backward(X, W, lab, lse, ignore_index=w.ignore_index,
                                         shift=w.shift, reduction=w.reduction)
        else:
            loss, lse, n_valid, dX, dW, status = F.chunked(
                X, W, lab, ignore_index=w.ignore_index, shift=w.shift, reduction=w.reduction)
            bstatus = status
        torch.cuda.synchronize()
        got = dict(loss=float(loss), lse=lse.double().cpu().numpy(), n_valid=int(n_valid),
                   status=int(status), bstatus=int(bstatus),
                   dX=dX.reshape(w.N, w.H).double().cpu().numpy(),
                   dW=dW[torch.from_numpy(rows).to(DEV)].double().cpu().numpy())
        del dX, dW
        check(w, got, dict(ref, dW=ref["dW"][rows]), what=f"widest {mode} {dtype}")


# ---------------------------------------------------------------------------
# full sizes
# ---------------------------------------------------------------------------
FULL = ["tiny_f32", "qwen2_7b_head", "qwen3_sft_batch", "long_context", "ragged_vocab"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_against_stored_oracle(name):
    path = os.path.join(GOLDEN, f"full_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_full_expected.py)")
    e = np.load(path)
    print(f"[full] {name}", flush=True)
    w = synth.workload(name)
    got = run(w)
    ref = dict(n_valid=int(e["n_valid"]), loss=float(e["loss"]), lse=e["lse"],
               dX=e["dx"], dW=e["dw"])
    check(w, got, ref, dx_rows=e["dx_rows"], dw_rows=e["dw_rows"], what=name)
    check_block_coverage(w, e)
    check_sampled_rows(w, got, e, what=name)
    # invariants on the whole outputs
    _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    assert np.all(got["dX"][~valid] == 0.0)
    # Rows of G sum to zero, so every column of dW sums to zero up to rounding:
    # G is stored with relative error u_g per entry and sum_v |G_iv| <= 2c, so
    # |sum_v dW[v, h]| <= 2 u_g c sum_i |X_ih| + u_out sum_v |dW[v, h]| (+ FP32).
    u = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -23
    c = 1.0 / got["n_valid"] if w.reduction == "mean" else 1.0
    Xv = w.X[valid].astype(np.float64)
    bound = 2 * u * c * np.abs(Xv).sum(axis=0) + u * np.abs(got["dW"]).sum(axis=0)
    colsum = np.abs(got["dW"].sum(axis=0))
    assert np.all(colsum <= 1.01 * bound + 1e-12), (colsum / bound).max()


@pytest.mark.parametrize("grad_dtype", [None, torch.float32])
@pytest.mark.parametrize("mode", ["recompute", "chunked"])
def test_dW_accumulates_over_micro_batches(mode, grad_dtype):
    """dW_accumulate = 1 adds the gradient to dW (gradient accumulation; a
    weight tied to the input embedding): two micro-batches sharing W give the
    oracle's summed dW."""
    wa = synth.workload("qwen2_7b_head", T=700, H=256, V=3001, seed=161)
    wb = synth.workload("qwen2_7b_head", T=500, H=256, V=3001, seed=162)
    wb.W = wa.W
    refs = [oracle.flce(w.X, w.W, w.labels, shift=w.shift) for w in (wa, wb)]
    dW = None
    for k, w in enumerate((wa, wb)):
        X, W, lab = to_device(w)
        if mode == "recompute":
            _, lse, _, _ = F.forward(X, W, lab, -100, w.shift, w.reduction)
            dX, dW, st = F.backward(X, W, lab, lse, shift=w.shift, reduction=w.reduction,
                                    grad_dtype=grad_dtype, dW=dW, accumulate=k > 0)
        else:
            _, _, _, dX, dW, st = F.chunked(X, W, lab, shift=w.shift, reduction=w.reduction,
                                            grad_dtype=grad_dtype, dW=dW, accumulate=k > 0)
    torch.cuda.synchronize()
    assert int(st) == 0
    want = refs[0]["dW"] + refs[1]["dW"]
    got = dW.double().cpu().numpy()
    assert oracle.cosine(got, want) >= 0.9999
    assert np.abs(got - want).max() <= 1e-2 * np.abs(want).max()
    gx = dX.reshape(wb.N, wb.H).double().cpu().numpy()
    assert oracle.cosine(gx, refs[1]["dX"]) >= 0.9999


@pytest.mark.parametrize("mode", ["recompute", "chunked"])
def test_full_size_fp32_gradients_accumulated_twice(mode):
    """The full Qwen2-7B-like head with FP32 gradient outputs, the same batch
    twice into one dW (dW_accumulate): the sampled dX rows equal the stored
    oracle's, the sampled dW rows twice the stored ones."""
    path = os.path.join(GOLDEN, "full_qwen2_7b_head.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_full_expected.py)")
    e = np.load(path)
    w = synth.workload("qwen2_7b_head")
    print(f"[full fp32 accumulate] {mode}", flush=True)
    X, W, lab = to_device(w)
    dW = None
    for k in range(2):
        if mode == "recompute":
            _, lse, _, st = F.forward(X, W, lab, w.ignore_index, w.shift, w.reduction)
            dX, dW, bst = F.backward(X, W, lab, lse, ignore_index=w.ignore_index,
                                     shift=w.shift, reduction=w.reduction,
                                     grad_dtype=torch.float32, dW=dW, accumulate=k > 0)
        else:
            _, _, _, dX, dW, st = F.chunked(X, W, lab, ignore_index=w.ignore_index,
                                            shift=w.shift, reduction=w.reduction,
                                            grad_dtype=torch.float32, dW=dW,
                                            accumulate=k > 0)
            bst = st
        torch.cuda.synchronize()
        assert int(st) == 0 and int(bst) == 0
    assert dX.dtype == torch.float32 and dW.dtype == torch.float32
    dXh = dX.reshape(w.N, w.H)[torch.from_numpy(e["dx_rows"]).to(DEV)].double().cpu().numpy()
    dWh = dW[torch.from_numpy(e["dw_rows"]).to(DEV)].double().cpu().numpy()
    for name, got, want in (("dX", dXh, e["dx"].astype(np.float64)),
                            ("dW", dWh, 2.0 * e["dw"].astype(np.float64))):
        assert oracle.cosine(got, want) >= 0.9999, name
        for q in range(len(want)):
            if not np.any(want[q]):
                assert not np.any(got[q]), (name, q)
                continue
            assert oracle.cosine(got[q], want[q]) >= 0.999, (name, q)
            assert np.abs(got[q] - want[q]).max() <= 1e-2 * np.abs(want[q]).max(), (name, q)


@pytest.mark.parametrize("mode", ["recompute", "chunked"])
def test_one_target_over_many_rows(mode):
    """Most rows share one target, so that target's rows span many
    256-position blocks of the sorted (target, row) order and its one-hot sum
    for dW is carried across blocks; the others are spread over the
    vocabulary.  dW and dX against the oracle, plus the softmax parts."""
    w = synth.make_workload("skewed", B=1, T=3000, H=136, V=777, dtype="bf16", seed=4242,
                            labels="uniform", mask="count", mask_arg=300, shift=False,
                            reduction="mean")
    rng = np.random.default_rng(5)
    lab = w.labels.reshape(-1)
    hot = rng.random(lab.shape) < 0.6
    lab[hot & (lab != w.ignore_index)] = 5
    print(f"[skewed] {mode} N={w.N} H={w.H} V={w.V}", flush=True)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index, reduction=w.reduction,
                      shift=w.shift, mode="global")
    got = run(w) if mode == "recompute" else run_chunked(w, chunk_rows=512)
    check(w, got, ref, what=f"skewed {mode}")
    g32 = run(w, grad_dtype=torch.float32) if mode == "recompute" else \
        run_chunked(w, grad_dtype=torch.float32, chunk_rows=512)
    sx, sw = soft_parts(w, g32["dX"], g32["dW"], ref["n_valid"])
    rx, rw = soft_parts(w, ref["dX"], ref["dW"], ref["n_valid"])
    cmin, ntol = soft_tolerance(w)
    for name, a, b in (("dX", sx, rx), ("dW", sw, rw)):
        assert oracle.cosine(a, b) >= cmin, name
        assert abs(np.linalg.norm(a) / np.linalg.norm(b) - 1.0) <= ntol, name
