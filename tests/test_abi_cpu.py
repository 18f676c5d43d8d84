"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/flce.h declares, sizes its workspace linearly in N (never
with N*V), and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

import lm_head_linear_flce_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_[a-z_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(F.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(F.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name, value in re.findall(r"#define (FLCE_[A-Z0-9_]+) (\d+)", text):
        assert getattr(F, name) == int(value), name


def test_status_strings():
    for code in range(0, 11):
        s = F.flce_status_string(code)
        assert s and s != "unknown status code"
    assert F.flce_status_string(1234) == "unknown status code"


@pytest.mark.parametrize("B,T,H,V", [(1, 8192, 3584, 152064), (2, 8192, 4096, 151936),
                                     (1, 32768, 2048, 152064), (1, 4099, 1024, 262147)])
def test_workspace_is_far_below_the_logits(B, T, H, V):
    ws = F.flce_workspace_size(B, T, H, V, F.FLCE_DTYPE_BF16)
    logits = B * T * V * 2
    assert 0 < ws < logits / 2
    # the vocabulary only enters through a bounded block: quadrupling V adds
    # at most the forward's per-range partials
    ws4 = F.flce_workspace_size(B, T, H, 4 * V, F.FLCE_DTYPE_BF16)
    assert ws4 <= ws + 64 * B * T * 8 + (1 << 20)


def test_workspace_grows_linearly_in_rows():
    w1 = F.flce_workspace_size(1, 4096, 2048, 152064, F.FLCE_DTYPE_BF16)
    w2 = F.flce_workspace_size(1, 8192, 2048, 152064, F.FLCE_DTYPE_BF16)
    w4 = F.flce_workspace_size(1, 16384, 2048, 152064, F.FLCE_DTYPE_BF16)
    assert w2 <= 2.2 * w1 and w4 <= 2.2 * w2


@pytest.mark.parametrize("args,code", [
    ((1, 16, 100, 50, F.FLCE_DTYPE_BF16), F.FLCE_ERR_ALIGN),      # H % 8
    ((1, 16, 128, 50, 7), F.FLCE_ERR_DTYPE),
    ((-1, 16, 128, 50, F.FLCE_DTYPE_BF16), F.FLCE_ERR_SHAPE),
    ((1, 16, 128, 0, F.FLCE_DTYPE_BF16), F.FLCE_ERR_SHAPE),
    ((1, 16, 0, 50, F.FLCE_DTYPE_BF16), F.FLCE_ERR_SHAPE),
])
def test_workspace_size_rejects(args, code):
    with pytest.raises(F.FlceError) as e:
        F.flce_workspace_size(*args)
    assert e.value.code == code


def test_workspace_size_null_out_pointer():
    lib = ctypes.CDLL(F.library_path())
    lib.flce_workspace_size.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_void_p]
    assert lib.flce_workspace_size(1, 8, 8, 8, 1, None) == F.FLCE_ERR_NULL


# Fake, aligned, never dereferenced device addresses: every call below must be
# rejected by the host checks, which run before any HIP call.
P = 1 << 20


def fwd(**kw):
    a = dict(X=P, W=2 * P, labels=3 * P, B=1, T=16, H=128, V=50, dtype=F.FLCE_DTYPE_BF16,
             ignore_index=-100, reduction=F.FLCE_REDUCTION_MEAN, shift=0, loss=4 * P,
             lse=5 * P, n_valid=0, status=0, workspace=6 * P, workspace_bytes=1 << 30,
             stream=0)
    a.update(kw)
    return F.flce_forward(*a.values())


def bwd(**kw):
    a = dict(X=P, W=2 * P, labels=3 * P, B=1, T=16, H=128, V=50, dtype=F.FLCE_DTYPE_BF16,
             ignore_index=-100, reduction=F.FLCE_REDUCTION_MEAN, shift=0, lse=5 * P,
             grad_scale=0, dX=7 * P, dW=8 * P, grad_dtype=F.FLCE_DTYPE_BF16, dW_accumulate=0,
             status=0, workspace=16 * P, workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return F.flce_backward(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(X=0), F.FLCE_ERR_NULL), (dict(W=0), F.FLCE_ERR_NULL),
    (dict(labels=0), F.FLCE_ERR_NULL), (dict(loss=0), F.FLCE_ERR_NULL),
    (dict(lse=0), F.FLCE_ERR_NULL), (dict(H=100), F.FLCE_ERR_ALIGN),
    (dict(X=P + 8), F.FLCE_ERR_ALIGN), (dict(dtype=3), F.FLCE_ERR_DTYPE),
    (dict(reduction=3), F.FLCE_ERR_REDUCTION), (dict(workspace=0), F.FLCE_ERR_WORKSPACE),
    (dict(workspace_bytes=64), F.FLCE_ERR_WORKSPACE), (dict(V=-5), F.FLCE_ERR_SHAPE),
])
def test_forward_host_checks(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dX=0), F.FLCE_ERR_NULL), (dict(dW=0), F.FLCE_ERR_NULL),
    (dict(lse=0), F.FLCE_ERR_NULL), (dict(grad_dtype=5), F.FLCE_ERR_DTYPE),
    (dict(dtype=F.FLCE_DTYPE_F32, grad_dtype=F.FLCE_DTYPE_BF16), F.FLCE_ERR_DTYPE),
    (dict(dX=P), F.FLCE_ERR_ALIAS), (dict(dW=2 * P + 64), F.FLCE_ERR_ALIAS),
    # dX is 16 x 128 bf16 = 4 KiB at 7 P; the workspace starts at 16 P
    (dict(dW=7 * P + 1024), F.FLCE_ERR_ALIAS), (dict(dX=16 * P + 4096), F.FLCE_ERR_ALIAS),
    (dict(dW=16 * P), F.FLCE_ERR_ALIAS),
    (dict(workspace_bytes=10), F.FLCE_ERR_WORKSPACE), (dict(reduction=9), F.FLCE_ERR_REDUCTION),
    (dict(dW=8 * P + 4), F.FLCE_ERR_ALIGN),
])
def test_backward_host_checks(kw, code):
    assert bwd(**kw) == code


def chk(**kw):
    a = dict(X=P, W=2 * P, labels=3 * P, B=1, T=16, H=128, V=50, dtype=F.FLCE_DTYPE_BF16,
             ignore_index=-100, reduction=F.FLCE_REDUCTION_MEAN, shift=0, chunk_rows=0,
             grad_scale=0, loss=4 * P, lse=5 * P, n_valid=0, dX=7 * P, dW=8 * P,
             grad_dtype=F.FLCE_DTYPE_BF16, dW_accumulate=0, status=0, workspace=16 * P,
             workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return F.flce_chunked(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(X=0), F.FLCE_ERR_NULL), (dict(W=0), F.FLCE_ERR_NULL),
    (dict(labels=0), F.FLCE_ERR_NULL), (dict(loss=0), F.FLCE_ERR_NULL),
    (dict(lse=0), F.FLCE_ERR_NULL), (dict(dX=0), F.FLCE_ERR_NULL),
    (dict(dW=0), F.FLCE_ERR_NULL), (dict(H=100), F.FLCE_ERR_ALIGN),
    (dict(X=P + 8), F.FLCE_ERR_ALIGN), (dict(dtype=3), F.FLCE_ERR_DTYPE),
    (dict(grad_dtype=5), F.FLCE_ERR_DTYPE), (dict(reduction=3), F.FLCE_ERR_REDUCTION),
    (dict(dX=P), F.FLCE_ERR_ALIAS), (dict(dW=2 * P + 64), F.FLCE_ERR_ALIAS),
    (dict(dW=7 * P + 1024), F.FLCE_ERR_ALIAS), (dict(dX=16 * P + 4096), F.FLCE_ERR_ALIAS),
    (dict(dW=16 * P), F.FLCE_ERR_ALIAS),
    (dict(workspace=0), F.FLCE_ERR_WORKSPACE), (dict(workspace_bytes=64), F.FLCE_ERR_WORKSPACE),
    (dict(V=-5), F.FLCE_ERR_SHAPE), (dict(chunk_rows=-1), F.FLCE_ERR_SHAPE),
])
def test_chunked_host_checks(kw, code):
    assert chk(**kw) == code


@pytest.mark.parametrize("args,code", [
    ((P, P, 64, 2 * P, 2 * P, 64, F.FLCE_DTYPE_BF16, 0, 0), F.FLCE_ERR_NULL),
    ((P, P, 63, 2 * P, 2 * P, 64, F.FLCE_DTYPE_F32, 3 * P, 0), F.FLCE_ERR_SHAPE),
    ((P, P, 64, 2 * P, 2 * P, 60, F.FLCE_DTYPE_BF16, 3 * P, 0), F.FLCE_ERR_SHAPE),
    ((P, P, 64, 2 * P, 2 * P, 64, 7, 3 * P, 0), F.FLCE_ERR_DTYPE),
    ((0, P, 64, 2 * P, 2 * P, 64, F.FLCE_DTYPE_BF16, 3 * P, 0), F.FLCE_ERR_NULL),
    ((P, 0, 64, 2 * P, 2 * P, 64, F.FLCE_DTYPE_BF16, 3 * P, 0), F.FLCE_ERR_NULL),
    ((P + 4, P + 4, 64, 2 * P, 2 * P, 64, F.FLCE_DTYPE_BF16, 3 * P, 0), F.FLCE_ERR_ALIGN),
    # an output overlapping its input without being it
    ((P, P + 16, 64, 2 * P, 2 * P, 64, F.FLCE_DTYPE_BF16, 3 * P, 0), F.FLCE_ERR_ALIAS),
    ((P, P, 64, 2 * P, 2 * P - 16, 64, F.FLCE_DTYPE_F32, 3 * P, 0), F.FLCE_ERR_ALIAS),
])
def test_scale_grads_host_checks(args, code):
    assert F.flce_scale_grads(*args) == code


def test_chunked_workspace_is_bounded_by_the_chunk():
    # the slab holds less than 2 GiB of one chunk's softmax gradient: beyond a
    # few thousand rows the workspace grows only by the per-row buffers
    H, V = 2048, 152064
    w1 = F.flce_chunked_workspace_size(1, 8192, H, V, F.FLCE_DTYPE_BF16)
    w2 = F.flce_chunked_workspace_size(1, 32768, H, V, F.FLCE_DTYPE_BF16)
    per_row = (w2 - w1) / (32768 - 8192)
    # per row: FP32 dX sum, compacted X copy, FP32 one-hot sum row for dW,
    # and a few words (sort key, indices, lse)
    assert per_row < 4 * H + 2 * H + 4 * H + 64
    # per chunk row (C = 6912 here): lse partials (16 bytes per vocabulary
    # tile), the scaled row X_s, at most one FP32 row of extra dX parts
    C = 6912
    assert w1 < (1 << 31) + 8192 * (10 * H + 64) + C * (16 * 594 + 6 * H) + (4 << 20) + 4 * V
    assert w2 < 32768 * V * 2                # far below the logits


def test_recompute_slabs_bounded():
    # the backward's two softmax-gradient slabs: 512 MiB, or up to 1 GiB where
    # that widens blocks toward 8192 columns (long context: 32768 rows get
    # 8192-column blocks, 1 GiB); never more, however many rows
    H, V, es = 2048, 152064, 2
    small = F.flce_workspace_size(1, 8192, H, V, F.FLCE_DTYPE_BF16)
    long_ = F.flce_workspace_size(1, 32768, H, V, F.FLCE_DTYPE_BF16)
    # beside the per-row buffers (FP32 dX sums, X_c, FP32 one-hot sums: 10 H
    # bytes, plus a few words), the slabs grew from 512 MiB to 1 GiB
    grown = long_ - small - (32768 - 8192) * (4 * H + H * es + 4 * H)
    assert (512 << 20) <= grown < (512 << 20) + (24 << 20)
    assert long_ < (1 << 30) + 32768 * (10 * H + 80) + (2048 * 256 * 8) + 4 * V + (8 << 20)
    huge = F.flce_workspace_size(1, 1 << 20, 1024, 32000, F.FLCE_DTYPE_BF16)
    assert huge < (1 << 30) + (1 << 20) * (4 * 1024 + 2 * 1024 + 4 * 1024 + 64 + 16) + (64 << 20)


def test_chunk_rows_past_the_2_31_byte_slab():
    # explicit chunks whose slab passes 2^31 bytes are accepted (each token
    # tile of the slab has its own 64-bit base); a vocabulary whose 256-row
    # slab tile passes 2^31 bytes is refused
    H, V = 4096, 151936
    vp = (V + 255) // 256 * 256
    w = F.flce_chunked_workspace_size(1, 16384, H, V, F.FLCE_DTYPE_BF16, 10240)
    assert w >= 10240 * vp * 2 > (1 << 31)
    for V, dt in ((4194048, F.FLCE_DTYPE_BF16), (2096896, F.FLCE_DTYPE_F32)):
        assert F.flce_chunked_workspace_size(1, 512, 64, V, dt) > 0
        with pytest.raises(F.FlceError) as e:
            F.flce_chunked_workspace_size(1, 512, 64, V + 1, dt)
        assert e.value.code == F.FLCE_ERR_SHAPE


def test_chunked_grid_within_a_dispatch():
    # one chunk of 2^22 - 256 rows over a 4194048-entry vocabulary would need
    # 2.7e8 logits workgroups, past a dispatch's 2^32 work items: refused
    # (whatever the memory, before any launch); the same rows in the default
    # chunks are planned
    N, V = 2 ** 22 - 256, 4194048
    with pytest.raises(F.FlceError) as e:
        F.flce_chunked_workspace_size(1, N, 8, V, F.FLCE_DTYPE_BF16, N)
    assert e.value.code == F.FLCE_ERR_SHAPE
    assert F.flce_chunked_workspace_size(1, N, 8, V, F.FLCE_DTYPE_BF16) > 0


def test_chunk_rows_parameter():
    # explicit chunk sizes round up to 256 rows; the slab is chunk x padded V
    H, V, es = 1024, 50000, 2
    vp = (V + 255) // 256 * 256
    w512 = F.flce_chunked_workspace_size(1, 8192, H, V, F.FLCE_DTYPE_BF16, 512)
    w300 = F.flce_chunked_workspace_size(1, 8192, H, V, F.FLCE_DTYPE_BF16, 300)
    w1024 = F.flce_chunked_workspace_size(1, 8192, H, V, F.FLCE_DTYPE_BF16, 1024)
    assert w300 == w512
    assert w1024 - w512 >= 512 * vp * es
    # at most the padded row count
    assert (F.flce_chunked_workspace_size(1, 1000, H, V, F.FLCE_DTYPE_BF16, 1 << 20)
            == F.flce_chunked_workspace_size(1, 1000, H, V, F.FLCE_DTYPE_BF16, 1024))


def sfwd(**kw):
    a = dict(X=P, W=2 * P, labels=3 * P, B=1, T=16, H=128, V=50, v_begin=10, V_total=100,
             dtype=F.FLCE_DTYPE_BF16, ignore_index=-100, shift=0, lse=5 * P, zt=4 * P,
             status=0, workspace=6 * P, workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return F.flce_shard_forward(*a.values())


def sbwd(**kw):
    a = dict(X=P, W=2 * P, labels=3 * P, B=1, T=16, H=128, V=50, v_begin=10, V_total=100,
             dtype=F.FLCE_DTYPE_BF16, ignore_index=-100, reduction=F.FLCE_REDUCTION_MEAN,
             shift=0, lse=5 * P, grad_scale=0, dX_partial=7 * P, dW=8 * P,
             grad_dtype=F.FLCE_DTYPE_BF16, dW_accumulate=0, status=0, workspace=16 * P,
             workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return F.flce_shard_backward(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(v_begin=60), F.FLCE_ERR_SHAPE), (dict(v_begin=-1), F.FLCE_ERR_SHAPE),
    (dict(V_total=40), F.FLCE_ERR_SHAPE), (dict(zt=0), F.FLCE_ERR_NULL),
    (dict(lse=0), F.FLCE_ERR_NULL), (dict(H=100), F.FLCE_ERR_ALIGN),
    (dict(workspace_bytes=64), F.FLCE_ERR_WORKSPACE),
])
def test_shard_forward_host_checks(kw, code):
    assert sfwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(v_begin=51), F.FLCE_ERR_SHAPE), (dict(dX_partial=0), F.FLCE_ERR_NULL),
    (dict(dW=0), F.FLCE_ERR_NULL), (dict(reduction=3), F.FLCE_ERR_REDUCTION),
    (dict(dX_partial=P), F.FLCE_ERR_ALIAS), (dict(grad_dtype=5), F.FLCE_ERR_DTYPE),
    (dict(dW=7 * P + 4096), F.FLCE_ERR_ALIAS), (dict(dX_partial=16 * P + 64), F.FLCE_ERR_ALIAS),
    (dict(workspace=0), F.FLCE_ERR_WORKSPACE),
])
def test_shard_backward_host_checks(kw, code):
    assert sbwd(**kw) == code


def test_shard_merge_host_checks():
    ws = F.flce_shard_merge_workspace_size(2, 1000)
    args = dict(lse_shards=P, zt_shards=2 * P, shards=3, labels=3 * P, B=2, T=1000,
                V_total=100, ignore_index=-100, shift=1, reduction=F.FLCE_REDUCTION_MEAN,
                loss=4 * P, lse=5 * P, n_valid=0, status=0, workspace=6 * P,
                workspace_bytes=ws, stream=0)
    for kw, code in ((dict(shards=0), F.FLCE_ERR_SHAPE), (dict(lse_shards=0), F.FLCE_ERR_NULL),
                     (dict(reduction=7), F.FLCE_ERR_REDUCTION),
                     (dict(workspace_bytes=ws - 1), F.FLCE_ERR_WORKSPACE)):
        a = dict(args)
        a.update(kw)
        assert F.flce_shard_merge(*a.values()) == code


def fwd_noalloc(**kw):
    a = dict(X=P, W=2 * P, labels=3 * P, B=1, T=16, H=128, V=50, dtype=F.FLCE_DTYPE_BF16,
             ignore_index=-100, reduction=F.FLCE_REDUCTION_MEAN, shift=0, loss=4 * P,
             lse=5 * P, n_valid=0, status=0, stream=0)
    a.update(kw)
    return F.flce_forward_noalloc(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(X=0), F.FLCE_ERR_NULL), (dict(loss=0), F.FLCE_ERR_NULL),
    (dict(lse=0), F.FLCE_ERR_NULL), (dict(H=100), F.FLCE_ERR_ALIGN),
    (dict(W=2 * P + 8), F.FLCE_ERR_ALIGN), (dict(dtype=3), F.FLCE_ERR_DTYPE),
    (dict(reduction=3), F.FLCE_ERR_REDUCTION), (dict(V=0), F.FLCE_ERR_SHAPE),
    # the forward of these needs more than the fixed scratch array holds
    (dict(B=1, T=32768, H=4096), F.FLCE_ERR_TOO_LARGE),
    (dict(B=2, T=1 << 20, H=64), F.FLCE_ERR_TOO_LARGE),
    (dict(B=1, T=65536, H=2048, dtype=F.FLCE_DTYPE_F32), F.FLCE_ERR_TOO_LARGE),
])
def test_forward_noalloc_host_checks(kw, code):
    assert fwd_noalloc(**kw) == code


@pytest.mark.parametrize("B,T,H,V,dt", [
    (1, 8192, 3584, 152064, F.FLCE_DTYPE_BF16), (2, 8192, 4096, 151936, F.FLCE_DTYPE_BF16),
    (1, 32768, 2048, 152064, F.FLCE_DTYPE_BF16), (1, 4099, 1024, 262147, F.FLCE_DTYPE_BF16),
    (2, 64, 256, 4096, F.FLCE_DTYPE_F32), (1, 1 << 20, 64, 1000, F.FLCE_DTYPE_BF16),
])
def test_forward_noalloc_fits_the_workloads(B, T, H, V, dt):
    # the stated bound: N * (H * es + 24) + 4 MiB <= the array's 160 MiB
    es = 2 if dt == F.FLCE_DTYPE_BF16 else 4
    assert B * T * (H * es + 24) + (4 << 20) <= F.FLCE_NOALLOC_SCRATCH_BYTES
    assert F.FLCE_NOALLOC_SCRATCH_BYTES == 160 << 20
    # NULL X passes the size check and fails the pointer check after it
    assert fwd_noalloc(B=B, T=T, H=H, V=V, dtype=dt, X=0) == F.FLCE_ERR_NULL


def test_noalloc_scratch_constant_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define FLCE_NOALLOC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == F.FLCE_NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("args,code", [
    ((P, 2 * P, 64, 9, 0, 0, 0), F.FLCE_ERR_DTYPE),
    ((P, 2 * P, 62, F.FLCE_DTYPE_BF16, 0, 0, 0), F.FLCE_ERR_SHAPE),
    ((P, 2 * P, -4, F.FLCE_DTYPE_BF16, 0, 0, 0), F.FLCE_ERR_SHAPE),
    ((0, 2 * P, 64, F.FLCE_DTYPE_BF16, 0, 0, 0), F.FLCE_ERR_NULL),
    ((P, 0, 64, F.FLCE_DTYPE_F32, 0, 0, 0), F.FLCE_ERR_NULL),
    ((P + 4, 2 * P, 64, F.FLCE_DTYPE_BF16, 0, 0, 0), F.FLCE_ERR_ALIGN),
    ((P, P + 128, 64, F.FLCE_DTYPE_BF16, 0, 0, 0), F.FLCE_ERR_ALIAS),
    ((P, 2 * P, 0, F.FLCE_DTYPE_BF16, 0, 0, 0), F.FLCE_OK),     # nothing to do
])
def test_convert_grads_host_checks(args, code):
    assert F.flce_convert_grads(*args) == code


@pytest.mark.parametrize("B,T,H,V", [(1, 262144, 4096, 151936), (1, 131072, 4096, 152064),
                                     (1, 65536, 8192, 152064), (8, 8192, 8192, 151936),
                                     (1, 1 << 20, 1024, 32000)])
def test_long_sequences_are_accepted(B, T, H, V):
    # N * H well past 2^29: the kernels address the FP32 sums per token tile
    # and, past 2^31 bytes of rows, rebase the dW loaders' descriptors per K
    # step, so only the workspace grows (linearly in N), never with N * V
    for dt in (F.FLCE_DTYPE_BF16, F.FLCE_DTYPE_F32):
        ws = F.flce_workspace_size(B, T, H, V, dt)
        assert 0 < ws < B * T * V * 2
        cws = F.flce_chunked_workspace_size(B, T, H, V, dt)
        assert 0 < cws < B * T * V * 2


def test_huge_vocabulary_recompute_only():
    # V past 2^24: the recompute path plans it (workspace linear in V for the
    # one-hot map, not in N * V); the chunked mode refuses it, as one 256-row
    # chunk of its [C, V] slab would pass 2^31 bytes
    V = 2 ** 24 + 43
    ws = F.flce_workspace_size(1, 256, 64, V, F.FLCE_DTYPE_BF16)
    assert 0 < ws < 256 * V * 2
    with pytest.raises(F.FlceError) as e:
        F.flce_chunked_workspace_size(1, 256, 64, V, F.FLCE_DTYPE_BF16)
    assert e.value.code == F.FLCE_ERR_SHAPE


def test_rows_bound_by_the_softmax_slab():
    # the narrowest vocabulary block (256 columns) of a rows_pad-row slab must
    # stay below 2^31 bytes: 2^22 - 256 bf16 rows pass, one more tile does not
    assert F.flce_workspace_size(1, 2 ** 22 - 256, 8, 300, F.FLCE_DTYPE_BF16) > 0
    with pytest.raises(F.FlceError) as e:
        F.flce_workspace_size(1, 2 ** 22, 8, 300, F.FLCE_DTYPE_BF16)
    assert e.value.code == F.FLCE_ERR_SHAPE
