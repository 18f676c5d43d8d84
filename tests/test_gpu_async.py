"""The calls are asynchronous on the caller's stream and never synchronise the
host: run on a non-default stream, and captured into a graph with a
preallocated workspace and outputs, they give bitwise the same loss, lse, dX
and dW as the eager calls on the default stream.  Graph replays are checked
one by one, with other eager work and synchronisations between them."""
import numpy as np
import pytest
import torch

import lm_head_linear_flce_amd as F
import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu


class Case:
    def __init__(self, w, chunked=False):
        self.w = w
        self.chunked = chunked
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.dc = F.FLCE_DTYPE_BF16 if w.dtype == "bf16" else F.FLCE_DTYPE_F32
        self.X = torch.from_numpy(w.X).to(DEV).to(dt)
        self.W = torch.from_numpy(w.W).to(DEV).to(dt)
        self.lab = torch.from_numpy(np.ascontiguousarray(w.labels)).to(DEV)
        self.red = {"mean": F.FLCE_REDUCTION_MEAN, "sum": F.FLCE_REDUCTION_SUM}[w.reduction]
        if chunked:
            self.nb = F.flce_chunked_workspace_size(w.B, w.T, w.H, w.V, self.dc, 512)
        else:
            self.nb = F.flce_workspace_size(w.B, w.T, w.H, w.V, self.dc)
        self.ws = torch.empty(self.nb, dtype=torch.uint8, device=DEV)
        self.gs = torch.tensor(1.5, dtype=torch.float32, device=DEV)
        self.out = dict(loss=torch.empty((), dtype=torch.float32, device=DEV),
                        lse=torch.empty(w.N, dtype=torch.float32, device=DEV),
                        dX=torch.empty(w.N, w.H, dtype=dt, device=DEV),
                        dW=torch.empty(w.V, w.H, dtype=dt, device=DEV))

    def poison(self):
        for t in self.out.values():
            t.fill_(float("nan"))

    def call(self, stream):
        w, o = self.w, self.out
        if self.chunked:
            rc = F.flce_chunked(self.X.data_ptr(), self.W.data_ptr(), self.lab.data_ptr(), w.B,
                                w.T, w.H, w.V, self.dc, w.ignore_index, self.red, w.shift, 512,
                                self.gs.data_ptr(), o["loss"].data_ptr(), o["lse"].data_ptr(),
                                0, o["dX"].data_ptr(), o["dW"].data_ptr(), self.dc, 0, 0,
                                self.ws.data_ptr(), self.nb, stream)
            assert rc == F.FLCE_OK, F.flce_status_string(rc)
            return
        rc = F.flce_forward(self.X.data_ptr(), self.W.data_ptr(), self.lab.data_ptr(), w.B, w.T,
                            w.H, w.V, self.dc, w.ignore_index, self.red, w.shift,
                            o["loss"].data_ptr(), o["lse"].data_ptr(), 0, 0, self.ws.data_ptr(),
                            self.nb, stream)
        assert rc == F.FLCE_OK, F.flce_status_string(rc)
        rc = F.flce_backward(self.X.data_ptr(), self.W.data_ptr(), self.lab.data_ptr(), w.B, w.T,
                             w.H, w.V, self.dc, w.ignore_index, self.red, w.shift,
                             o["lse"].data_ptr(), self.gs.data_ptr(), o["dX"].data_ptr(),
                             o["dW"].data_ptr(), self.dc, 0, 0, self.ws.data_ptr(), self.nb,
                             stream)
        assert rc == F.FLCE_OK, F.flce_status_string(rc)

    def snapshot(self):
        return {k: v.clone() for k, v in self.out.items()}


def _bitwise_equal(a, b):
    for k in a:
        x, y = a[k], b[k]
        assert x.shape == y.shape, k
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)), k


def _workloads():
    return [synth.workload("qwen2_7b_head", T=1100, H=264, V=9001, seed=3101),
            synth.workload("ragged_vocab", T=900, H=200, V=7001, seed=3102)]


@pytest.mark.parametrize("chunked", [False, True])
def test_non_default_stream_matches_default(chunked):
    for w in _workloads():
        c = Case(w, chunked)
        c.poison()
        c.call(0)
        torch.cuda.synchronize()
        ref = c.snapshot()
        s = torch.cuda.Stream()
        c.poison()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            c.call(s.cuda_stream)
        s.synchronize()
        _bitwise_equal(ref, c.out)
        assert torch.isfinite(ref["loss"]).item()


@pytest.mark.parametrize("chunked", [False, True])
def test_graph_capture_replays_match_eager(chunked):
    w, other = _workloads()
    c, d = Case(w, chunked), Case(other, chunked)
    c.call(0)
    torch.cuda.synchronize()
    ref = c.snapshot()
    d.call(0)
    torch.cuda.synchronize()
    ref_d = d.snapshot()
    # warm up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c.call(s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.call(torch.cuda.current_stream().cuda_stream)
    for r in range(3):
        c.poison()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] chunked={chunked} replay {r}", flush=True)
        _bitwise_equal(ref, c.out)
        # other eager work between the replays, on the same device
        d.poison()
        d.call(0)
        torch.cuda.synchronize()
        _bitwise_equal(ref_d, d.out)
