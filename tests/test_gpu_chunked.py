"""Parity of the chunked mode (flce_chunked: loss, lse, dX, dW in one call over
row chunks) with the float64 oracle, through the C ABI.

The oracle is the same plain definition as for the forward / backward pair;
the chunked schedule must reach the same result (the ms-swift PR "feat(sft):
Add optional fused linear ce for qwen2/qwen3 on npu", "Mathematical
Equivalence")."""
import os

import numpy as np
import pytest
import torch

import lm_head_linear_flce_amd as F
import oracle
import synth
from gpu_util import (DEV, check, check_block_coverage, check_sampled_rows, run,
                      run_chunked, soft_parts, soft_tolerance, to_device)
from test_gpu_parity import GOLDEN, SMALL, _ids

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", SMALL, ids=[_ids(p) for p in SMALL])
def test_chunked_small_parity(case):
    name, ov = case
    w = synth.workload(name, **ov)
    print(f"[chunked] {name} {ov} N={w.N} H={w.H} V={w.V}", flush=True)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="rows", chunk=1024)
    got = run_chunked(w)
    check(w, got, ref, what="chunked " + name)
    _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    assert np.all(got["dX"][~valid] == 0.0)


@pytest.mark.parametrize("case", SMALL[:5], ids=[_ids(p) for p in SMALL[:5]])
def test_chunked_softmax_part_of_the_gradients(case):
    """As for the recompute path: the softmax parts P W and P^T X, rebuilt from
    the FP32 gradient outputs, in direction and size."""
    name, ov = case
    w = synth.workload(name, **ov)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="rows", chunk=1024)
    got = run_chunked(w, grad_dtype=torch.float32)
    n = ref["n_valid"]
    gx, gw = soft_parts(w, got["dX"], got["dW"], n)
    rx, rw = soft_parts(w, ref["dX"], ref["dW"], n)
    cx, cw = oracle.cosine(gx, rx), oracle.cosine(gw, rw)
    print(f"[chunked soft part] {name}: cos P.W {cx:.7f}  cos P^T.X {cw:.7f}", flush=True)
    rnx = np.linalg.norm(gx) / np.linalg.norm(rx)
    rnw = np.linalg.norm(gw) / np.linalg.norm(rw)
    # fp32 G: the soft parts to rounding; bf16 G: see soft_tolerance
    cmin, rtol = soft_tolerance(w)
    assert cx >= cmin and cw >= cmin, (cx, cw)
    assert abs(rnx - 1) <= rtol and abs(rnw - 1) <= rtol, (rnx, rnw)


def test_chunked_several_chunks():
    # V large enough that the default [C, V] slab (under 2^31 bytes: 3840
    # rows at V = 262147) holds fewer rows than there are valid rows: dW is
    # summed over two chunks, a full one and a short last one
    w = synth.workload("qwen2_7b_head", T=5003, H=64, V=262147, seed=201)
    print(f"[chunked] several chunks N={w.N} V={w.V}", flush=True)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="rows", chunk=512)
    vp = (w.V + 255) // 256 * 256
    assert ref["n_valid"] > ((1 << 31) - 1) // (vp * 2) // 256 * 256
    got = run_chunked(w)
    check(w, got, ref, what="chunked several")
    got32 = run_chunked(w, grad_dtype=torch.float32)
    check(w, got32, ref, what="chunked several fp32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_short_last_chunk_takes_more_dx_parts(dtype):
    """2100 rows in chunks of 1024: the last chunk holds 52 rows (one token
    tile) and cuts its dX tiles into 8 vocabulary parts where the full chunks
    (8 hidden x 4 token tiles) use 6, inside the same part buffer; every part
    is summed once, in order, into that chunk's rows."""
    w = synth.make_workload("short_last_chunk", B=1, T=2100, H=2048, V=3001, dtype=dtype,
                            seed=919, shift=False, reduction="mean")
    print(f"[chunked] short last chunk {dtype} N={w.N} H={w.H} V={w.V}", flush=True)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="rows", chunk=1024)
    assert ref["n_valid"] == 2100
    check(w, run_chunked(w, chunk_rows=1024), ref, what=f"short last chunk {dtype}")
    check(w, run_chunked(w, chunk_rows=1024, grad_dtype=torch.float32), ref,
          what=f"short last chunk {dtype} fp32 grads")


@pytest.mark.parametrize("chunk_rows", [256, 700])
def test_chunked_explicit_chunk_rows(chunk_rows):
    # the pages' CHUNK_SIZE knob: many small chunks give the same result
    w = synth.workload("qwen3_sft_batch", T=1500, H=392, V=5003, seed=37)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="rows", chunk=1024)
    assert ref["n_valid"] > 768
    check(w, run_chunked(w, chunk_rows=chunk_rows), ref, what=f"chunk_rows={chunk_rows}")
    check(w, run_chunked(w, chunk_rows=chunk_rows, grad_dtype=torch.float32), ref,
          what=f"chunk_rows={chunk_rows} fp32")


@pytest.mark.parametrize("case", SMALL[2:4], ids=[_ids(p) for p in SMALL[2:4]])
def test_chunked_matches_recompute_path(case):
    """Same loss / lse as the forward; gradients agree to bf16 rounding."""
    name, ov = case
    w = synth.workload(name, **ov)
    a = run(w)
    b = run_chunked(w)
    assert abs(a["loss"] - b["loss"]) <= 1e-5 * abs(a["loss"])
    np.testing.assert_allclose(b["lse"], a["lse"], rtol=0, atol=2e-5)
    for k in ("dX", "dW"):
        assert oracle.cosine(a[k], b[k]) > 0.9999


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunked_logits_far_from_zero(dtype):
    """Rows whose logits sit near +-120 (beyond the +-44 the slab's fixed
    reference covers, so they are stored again against their own max) next to
    rows near zero, over several chunks: loss, lse and both gradients against
    the oracle, and the same results as the recompute path."""
    w = synth.far_logit_workload(B=1, T=1100, H=256, V=3001, dtype=dtype, seed=881)
    print(f"[chunked far logits] {dtype} N={w.N} H={w.H} V={w.V}", flush=True)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index,
                      reduction=w.reduction, shift=w.shift, mode="rows", chunk=1024)
    assert np.abs(ref["lse"]).max() > 80.0 and np.abs(ref["lse"]).min() < 20.0
    got = run_chunked(w, chunk_rows=256)
    # |lse| up to ~140: the FP32 logits' own rounding over H = 256 terms is
    # ~sqrt(H) ulp(140) ~ 1e-4, so the lse bound grows with |lse| (4e-6 |lse|)
    check(w, got, ref, what="chunked far logits " + dtype, lse_rel=4e-6)
    a = run(w)
    assert abs(a["loss"] - got["loss"]) <= 1e-5 * abs(a["loss"])
    for k in ("dX", "dW"):
        assert oracle.cosine(a[k], got[k]) > 0.9999


def test_chunked_autograd_and_grad_scale():
    w = synth.workload("qwen2_7b_head", T=300, H=128, V=700, seed=71)
    X, W, lab = to_device(w)
    Xr = X.detach().clone().requires_grad_(True)
    Wr = W.detach().clone().requires_grad_(True)
    loss = F.linear_cross_entropy(Xr, Wr, lab, ignore_index=-100, shift=True,
                                  reduction="mean", mode="chunked")
    (2.5 * loss).backward()
    ref = oracle.flce(w.X, w.W, w.labels, shift=True, grad_scale=2.5)
    assert abs(float(loss.detach()) - ref["loss"]) <= 2e-3 * abs(ref["loss"])
    gx = Xr.grad.reshape(w.N, w.H).double().cpu().numpy()
    gw = Wr.grad.double().cpu().numpy()
    assert oracle.cosine(gx, ref["dX"]) >= 0.9999
    assert oracle.cosine(gw, ref["dW"]) >= 0.9999
    # the scale inside the call gives the same gradients
    got = run_chunked(w, grad_scale=2.5)
    assert oracle.cosine(got["dW"], ref["dW"]) >= 0.9999


def test_chunked_autograd_second_backward():
    """A second backward through a retained graph gets the same gradients: the
    saved unit-scale gradients are scaled out of place, not in place."""
    w = synth.workload("qwen2_7b_head", T=300, H=128, V=700, seed=73)
    X, W, lab = to_device(w)
    Xr = X.detach().clone().requires_grad_(True)
    Wr = W.detach().clone().requires_grad_(True)
    loss = F.linear_cross_entropy(Xr, Wr, lab, ignore_index=-100, shift=True,
                                  reduction="mean", mode="chunked")
    g1 = torch.autograd.grad(2.0 * loss, (Xr, Wr), retain_graph=True)
    g2 = torch.autograd.grad(2.0 * loss, (Xr, Wr))
    ref = oracle.flce(w.X, w.W, w.labels, shift=True, grad_scale=2.0)
    for g in (g1, g2):
        assert oracle.cosine(g[0].reshape(w.N, w.H).double().cpu().numpy(), ref["dX"]) >= 0.9999
        assert oracle.cosine(g[1].double().cpu().numpy(), ref["dW"]) >= 0.9999
        rx = np.linalg.norm(g[1].double().cpu().numpy()) / np.linalg.norm(ref["dW"])
        assert abs(rx - 1.0) <= 1e-2
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1])


def test_chunked_no_valid_rows_and_bad_label():
    w = synth.workload("long_context", T=500, H=64, V=300, seed=101)
    w.labels[:] = -100
    got = run_chunked(w)
    assert got["n_valid"] == 0 and got["loss"] == 0.0
    assert not got["dX"].any() and not got["dW"].any() and not got["lse"].any()
    w = synth.workload("ragged_vocab", T=300, H=64, V=500, seed=121)
    w.labels[0, 5] = w.V + 3
    got = run_chunked(w)
    assert got["status"] == F.FLCE_ERR_LABEL_RANGE
    assert np.isnan(got["loss"]) and np.isnan(got["dW"]).any()


def test_chunked_is_bitwise_deterministic():
    w = synth.workload("ragged_vocab", T=900, H=256, V=3001, seed=81)
    outs = [run_chunked(w) for _ in range(2)]
    assert outs[0]["loss"] == outs[1]["loss"]
    for k in ("lse", "dX", "dW"):
        assert np.array_equal(outs[0][k], outs[1][k])


FULL = ["tiny_f32", "qwen2_7b_head", "qwen3_sft_batch", "long_context", "ragged_vocab"]


@pytest.mark.parametrize("grad_dtype", [None, torch.float32])
@pytest.mark.parametrize("name", FULL)
def test_full_size_chunked_against_stored_oracle(name, grad_dtype):
    """The chunked mode at the full sizes on the oracle's stored values (loss,
    every row's lse, sampled dX and dW rows); with bf16 outputs dW is rounded
    once per chunk (4 chunks for the long-context workload), with float32 the
    sum over the chunks stays FP32."""
    path = os.path.join(GOLDEN, f"full_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_full_expected.py)")
    e = np.load(path)
    print(f"[full chunked] {name}", flush=True)
    w = synth.workload(name)
    got = run_chunked(w, grad_dtype=grad_dtype)
    ref = dict(n_valid=int(e["n_valid"]), loss=float(e["loss"]), lse=e["lse"],
               dX=e["dx"], dW=e["dw"])
    check(w, got, ref, dx_rows=e["dx_rows"], dw_rows=e["dw_rows"], what="chunked " + name)
    check_block_coverage(w, e)
    check_sampled_rows(w, got, e, what="chunked " + name)
    _, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    assert np.all(got["dX"][~valid] == 0.0)


@pytest.mark.parametrize("name,chunk_rows", [("qwen3_sft_batch", 10240),
                                             ("long_context", 24576)])
def test_full_size_one_chunk_slab_past_2_31_bytes(name, chunk_rows):
    """All valid rows in one chunk whose softmax slab passes 2^31 bytes (3.1 GB
    for the Qwen3 batch, 7.5 GB, past 2^32, at long context): every token
    tile of the slab is stored and read from its own 64-bit base, against the
    oracle's stored values at the full size."""
    path = os.path.join(GOLDEN, f"full_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_full_expected.py)")
    e = np.load(path)
    w = synth.workload(name)
    vp = (w.V + 255) // 256 * 256
    assert int(e["n_valid"]) <= chunk_rows and chunk_rows * vp * 2 > (1 << 31)
    print(f"[full chunked, one chunk] {name} chunk_rows={chunk_rows}", flush=True)
    got = run_chunked(w, chunk_rows=chunk_rows)
    ref = dict(n_valid=int(e["n_valid"]), loss=float(e["loss"]), lse=e["lse"],
               dX=e["dx"], dW=e["dw"])
    check(w, got, ref, dx_rows=e["dx_rows"], dw_rows=e["dw_rows"],
          what=f"chunked {name} one chunk")
    check_sampled_rows(w, got, e, what=f"chunked {name} one chunk")


def test_round_once_over_many_chunks():
    """bf16 gradients over many row chunks: with round_once the chunked mode
    keeps dW in FP32 across the chunks and rounds once, so it matches the
    recompute path (one rounding of an FP32 sum over all rows) to the last
    bf16 bit up to summation order, and it is closer to the oracle than
    rounding once per chunk."""
    w = synth.workload("long_context", T=4096, H=256, V=20011, seed=4501)
    print(f"[round-once] N={w.N} H={w.H} V={w.V}, 512-row chunks", flush=True)
    ref = oracle.flce(w.X, w.W, w.labels, ignore_index=w.ignore_index, reduction=w.reduction,
                      shift=w.shift, mode="rows", chunk=1024)
    X, W, lab = to_device(w)
    once = F.chunked(X, W, lab, ignore_index=w.ignore_index, shift=w.shift,
                     reduction=w.reduction, chunk_rows=512, round_once=True)
    per_chunk = F.chunked(X, W, lab, ignore_index=w.ignore_index, shift=w.shift,
                          reduction=w.reduction, chunk_rows=512)
    rec = run(w)
    torch.cuda.synchronize()
    dw_once = once[4].double().cpu().numpy()
    dw_per = per_chunk[4].double().cpu().numpy()
    dx_once = once[3].reshape(w.N, w.H).double().cpu().numpy()
    assert once[4].dtype == torch.bfloat16 and once[3].dtype == torch.bfloat16
    # the recompute path forms G from exp(z - lse) and the chunked mode from a
    # per-tile exponent rescaled afterwards, so their bf16 G entries differ
    # by rounding: agreement in norm, not bit for bit
    for a, b in ((dw_once, rec["dW"]), (dx_once, rec["dX"])):
        assert np.linalg.norm(a - b) <= 2.0 ** -8 * np.linalg.norm(b)
        assert oracle.cosine(a, b) >= 0.99999
    # and closer to the oracle than one rounding per chunk
    e_once = np.linalg.norm(dw_once - ref["dW"])
    e_per = np.linalg.norm(dw_per - ref["dW"])
    print(f"[round-once] |dW - oracle|: once {e_once:.3e}, per chunk {e_per:.3e}", flush=True)
    assert e_once < e_per
    assert oracle.cosine(dw_once, ref["dW"]) >= 0.9999
