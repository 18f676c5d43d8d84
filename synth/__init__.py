"""Seeded synthetic inputs for the fused linear cross-entropy engine.

This module only draws numbers: hidden states X [N, H], an output weight W [V, H]
and integer labels [B, T].  It holds none of the loss arithmetic, and it is the
one piece shared by the float64 oracle (tests) and the GPU path (tests, bench).

The pages name no dataset for the fused loss (the LoRA-SFT blog post tokenises an
unnamed corpus with ``labels = input_ids``), so every input here is synthetic:
Gaussian hidden states (optionally RMS-normalised, as a final norm layer would
leave them), Gaussian output weights, and labels that are either uniform or
Zipf-distributed token ids, with masked prompt positions set to ``ignore_index``.

Recipe (fixed, so that any run can regenerate the same bytes):
  * generator: numpy PCG64 seeded with ``seed``; draw order X, W, labels, mask;
  * X ~ N(0, 1) as float32, then optionally x / sqrt(mean(x^2) + 1e-6) per row
    (computed in float64, stored float32);
  * W ~ N(0, w_std^2) as float32;
  * labels: uniform over [0, V), or Zipf(s) over ranks 1..V mapped to token ids
    through a seeded permutation (permutation drawn first, then the uniforms);
  * mask kinds: 'count' (exactly m flat positions, chosen without replacement),
    'prefix' (first m positions of every sequence), 'span' (one contiguous span
    per sequence of length L ~ U{lo..hi} starting at U{0..T-L});
  * bf16 inputs are rounded from float32 with round-to-nearest-even, and the same
    rounded values are handed to both sides.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

IGNORE_INDEX = -100


@dataclasses.dataclass
class Workload:
    """One synthetic problem. X and W hold float32 values; for dtype 'bf16' every
    value is exactly representable in bfloat16."""
    name: str
    X: np.ndarray          # [N, H] float32
    W: np.ndarray          # [V, H] float32
    labels: np.ndarray     # [B, T] int64
    B: int
    T: int
    H: int
    V: int
    dtype: str             # 'bf16' or 'f32'
    shift: bool
    reduction: str         # 'mean' or 'sum'
    ignore_index: int = IGNORE_INDEX

    @property
    def N(self) -> int:
        return self.B * self.T


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bfloat16 value, returned as float32 (finite input)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _normal(rng, shape, std):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _rms_normalise(x):
    out = np.empty_like(x)
    step = 4096
    for i in range(0, x.shape[0], step):
        blk = x[i:i + step].astype(np.float64)
        blk /= np.sqrt(np.mean(blk * blk, axis=1, keepdims=True) + 1e-6)
        out[i:i + step] = blk.astype(np.float32)
    return out


def _zipf_labels(rng, n, V, s):
    perm = rng.permutation(V).astype(np.int64)
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    rank = np.searchsorted(cdf, u, side="right")
    rank = np.minimum(rank, V - 1)
    return perm[rank]


def _mask(rng, labels, kind, arg, ignore_index):
    B, T = labels.shape
    if kind is None:
        return labels
    lab = labels.copy()
    if kind == "count":
        pos = rng.choice(B * T, size=int(arg), replace=False)
        lab.reshape(-1)[pos] = ignore_index
    elif kind == "prefix":
        lab[:, :int(arg)] = ignore_index
    elif kind == "span":
        lo, hi = arg
        for b in range(B):
            L = int(rng.integers(lo, hi + 1))
            s0 = int(rng.integers(0, T - L + 1))
            lab[b, s0:s0 + L] = ignore_index
    else:
        raise ValueError(f"unknown mask kind {kind!r}")
    return lab


def make_workload(name, *, B, T, H, V, dtype, seed, x_rms=False, w_std=0.02,
                  labels="uniform", zipf_s=1.1, mask=None, mask_arg=None,
                  shift=False, reduction="mean", ignore_index=IGNORE_INDEX):
    rng = np.random.Generator(np.random.PCG64(seed))
    N = B * T
    X = _normal(rng, (N, H), 1.0)
    if x_rms:
        X = _rms_normalise(X)
    W = _normal(rng, (V, H), w_std)
    if labels == "uniform":
        lab = rng.integers(0, V, size=N, dtype=np.int64)
    elif labels == "zipf":
        lab = _zipf_labels(rng, N, V, zipf_s)
    else:
        raise ValueError(f"unknown label distribution {labels!r}")
    lab = _mask(rng, lab.reshape(B, T), mask, mask_arg, ignore_index)
    if dtype == "bf16":
        X = round_to_bf16(X)
        W = round_to_bf16(W)
    elif dtype != "f32":
        raise ValueError(dtype)
    return Workload(name=name, X=X, W=W, labels=lab, B=B, T=T, H=H, V=V,
                    dtype=dtype, shift=shift, reduction=reduction,
                    ignore_index=ignore_index)


def far_logit_workload(*, B, T, H, V, dtype, seed, offset=120.0, w_std=0.05):
    """Logits far from zero: every W row carries a shared unit direction u, and
    row k of X carries t_k u with t_k uniform in [-offset, offset], so row k's
    logits sit around t_k (a spread of about w_std * sqrt(H) around it).  For
    schedules that keep exp(z) against a fixed reference: rows well above,
    well below and near zero in one problem."""
    rng = np.random.Generator(np.random.PCG64(seed))
    N = B * T
    u = _normal(rng, (H,), 1.0)
    u /= np.float32(np.linalg.norm(u.astype(np.float64)))
    W = _normal(rng, (V, H), w_std) + u[None, :]
    t = rng.uniform(-offset, offset, size=N).astype(np.float32)
    X = _normal(rng, (N, H), 1.0) + t[:, None] * u[None, :]
    lab = rng.integers(0, V, size=(B, T), dtype=np.int64)
    if dtype == "bf16":
        X = round_to_bf16(X)
        W = round_to_bf16(W)
    elif dtype != "f32":
        raise ValueError(dtype)
    return Workload(name="far_logits", X=X, W=W, labels=lab, B=B, T=T, H=H, V=V,
                    dtype=dtype, shift=False, reduction="mean", ignore_index=IGNORE_INDEX)


# The five workloads.  Sizes follow the LM heads the pages talk about: a ~152K
# token vocabulary (Qwen2/Qwen3 tokenizers), 8K-32K token sequences, hidden
# widths 1024-4096, and one prime-sized vocabulary to exercise ragged tiles.
WORKLOADS = {
    "tiny_f32": dict(B=2, T=64, H=256, V=4096, dtype="f32", seed=1001,
                     w_std=0.02, labels="uniform", mask="count",
                     mask_arg=13, shift=False, reduction="mean"),
    "qwen2_7b_head": dict(B=1, T=8192, H=3584, V=152064, dtype="bf16",
                          seed=1002, x_rms=True, w_std=0.02, labels="zipf",
                          mask="prefix", mask_arg=1638, shift=True,
                          reduction="mean"),
    "qwen3_sft_batch": dict(B=2, T=8192, H=4096, V=151936, dtype="bf16",
                            seed=1003, x_rms=True, w_std=0.02, labels="zipf",
                            mask="span", mask_arg=(math.ceil(0.3 * 8192),
                                                   math.floor(0.6 * 8192)),
                            shift=True, reduction="mean"),
    "long_context": dict(B=1, T=32768, H=2048, V=152064, dtype="bf16",
                         seed=1004, x_rms=True, w_std=0.02, labels="zipf",
                         mask="prefix", mask_arg=8192, shift=True,
                         reduction="mean"),
    "ragged_vocab": dict(B=1, T=4099, H=1024, V=262147, dtype="bf16",
                         seed=1005, w_std=0.05, labels="uniform",
                         mask="count", mask_arg=2049, shift=False,
                         reduction="sum"),
}


def workload(name: str, **override) -> Workload:
    """Build a named workload; keyword overrides (e.g. smaller T/H/V) keep the
    rest of the recipe, which gives same-shaped, oracle-sized variants."""
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    T = cfg["T"]
    # masks given as fractions of the sequence are rescaled with T
    if "T" in override and cfg["mask"] == "prefix":
        frac = WORKLOADS[name]["mask_arg"] / WORKLOADS[name]["T"]
        cfg["mask_arg"] = int(math.floor(frac * T))
    if "T" in override and cfg["mask"] == "span":
        cfg["mask_arg"] = (math.ceil(0.3 * T), math.floor(0.6 * T))
    if ("T" in override or "B" in override) and cfg["mask"] == "count" \
            and "mask_arg" not in override:
        frac = WORKLOADS[name]["mask_arg"] / (WORKLOADS[name]["B"] * WORKLOADS[name]["T"])
        cfg["mask_arg"] = int(math.floor(frac * cfg["B"] * T))
    return make_workload(name, **cfg)
