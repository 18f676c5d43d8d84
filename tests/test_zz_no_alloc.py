"""flce_forward_noalloc (the forward on the library's fixed device array, for
callers that cannot allocate) against flce_forward on the caller's workspace:
the same kernels on the same inputs, so loss, lse, n_valid and status must be
bitwise equal.  Two calls in a row share the array, the second smaller, so a
second call must not see the first one's leftovers."""
import numpy as np
import pytest
import torch

import lm_head_linear_flce_amd as F
import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def _both(w):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dcode = F.FLCE_DTYPE_BF16 if w.dtype == "bf16" else F.FLCE_DTYPE_F32
    X = torch.from_numpy(w.X).to(DEV).to(dt)
    W = torch.from_numpy(w.W).to(DEV).to(dt)
    lab = torch.from_numpy(np.ascontiguousarray(w.labels)).to(DEV)
    red = {"mean": F.FLCE_REDUCTION_MEAN, "sum": F.FLCE_REDUCTION_SUM}[w.reduction]
    stream = int(torch.cuda.current_stream().cuda_stream)
    outs = []
    for noalloc in (False, True):
        loss = torch.full((), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((w.N,), float("nan"), dtype=torch.float32, device=DEV)
        nv = torch.full((), -1, dtype=torch.int64, device=DEV)
        st = torch.full((), -1, dtype=torch.int32, device=DEV)
        args = (X.data_ptr(), W.data_ptr(), lab.data_ptr(), w.B, w.T, w.H, w.V, dcode,
                w.ignore_index, red, w.shift, loss.data_ptr(), lse.data_ptr(), nv.data_ptr(),
                st.data_ptr())
        if noalloc:
            rc = F.flce_forward_noalloc(*args, stream)
        else:
            nbytes = F.flce_workspace_size(w.B, w.T, w.H, w.V, dcode)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
            rc = F.flce_forward(*args, ws.data_ptr(), nbytes, stream)
        assert rc == F.FLCE_OK, F.flce_status_string(rc)
        torch.cuda.synchronize()
        outs.append((loss.cpu(), lse.cpu(), nv.cpu(), st.cpu()))
    return outs


def _same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x, y) or (x.dtype.is_floating_point and
                                     torch.equal(x.view(torch.int32), y.view(torch.int32)))


def test_noalloc_forward_matches_workspace_forward_twice():
    big = synth.workload("qwen2_7b_head", T=4096, H=1024, V=30011, seed=901)
    small = synth.workload("ragged_vocab", T=700, H=256, V=5003, seed=902)
    print("[noalloc] call 1: N=4096 H=1024 V=30011 bf16 shift mean", flush=True)
    ref, got = _both(big)
    _same(ref, got)
    assert int(got[3]) == 0 and int(got[2]) == int(ref[2])
    print("[noalloc] call 2: N=700 H=256 V=5003 bf16 sum", flush=True)
    ref, got = _both(small)
    _same(ref, got)
    assert np.isfinite(float(got[0]))


def test_noalloc_forward_full_size_head():
    w = synth.workload("qwen2_7b_head")
    print("[noalloc] N=8192 H=3584 V=152064 bf16", flush=True)
    ref, got = _both(w)
    _same(ref, got)
    assert int(got[2]) == 6554
