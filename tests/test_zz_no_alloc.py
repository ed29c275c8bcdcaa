"""The allocation-free block call (atom_attn_block_noalloc, scratch in the
library's static per-device array) against the workspace call
(atom_attn_encoder / atom_attn_decoder) through the C ABI: same kernels, so
the outputs must agree, on two calls in a row, the second with a smaller
input (the static array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from _parity import RTOL, assert_close, assert_close_rel, np64
from windowed_atom_attention_amd import (noalloc_max_bytes, windowed_atom_attention,
                                         workspace_bytes)
from windowed_atom_attention_amd import _native as N
from windowed_atom_attention_amd.workloads import make_workload

pytestmark = pytest.mark.gpu

CASES = [
    # (first call, second smaller call)
    (("1", dict(A=2000)), ("1", dict(A=700))),
    (("3", dict(B=2, A=1500)), ("3", dict(B=1, A=900))),
    (("2", dict(A=1800)), ("0", dict(style="esmfold2", dtype=torch.bfloat16))),
    (("4a", dict(A=3000, stage="decoder")), ("4b", dict(A=1000))),
]


def _outs(w):
    d = w.dims
    dev = "cuda"
    out = {"hidden": torch.empty((d["B"], d["A"], d["C"]), dtype=w.dtype, device=dev),
           "attention": torch.empty((d["B"], d["H"], d["A"], d["K"]), dtype=w.dtype,
                                    device=dev)}
    if w.stage == "encoder":
        out["token_output"] = torch.empty((d["B"], d["T"], d["U"]), dtype=w.dtype, device=dev)
    else:
        out["position_update"] = torch.empty((d["B"], d["A"], 3), dtype=w.dtype, device=dev)
    return out


def _check(w, got, ref):
    rtol = RTOL[w.dtype]
    for k in ref:
        g, r = np64(got[k]), np64(ref[k])
        # same kernels on the same inputs: identical bits
        assert np.array_equal(g, r), k
        if k == "attention":
            assert_close_rel(k, g, r, rtol)
        else:
            assert_close(k, g, r, rtol)


@pytest.mark.parametrize("case", CASES, ids=["%s-%s" % (a[0], b[0]) for a, b in CASES])
def test_noalloc_matches_workspace_call(case):
    for name, kw in case:
        w = make_workload(name, **kw)
        print("noalloc case", name, kw, w.dims, flush=True)
        assert workspace_bytes(w.dims, w.style, w.stage, w.dtype) <= noalloc_max_bytes()
        g = w.to("cuda")
        ref = windowed_atom_attention(**g.kwargs())
        # poison the outputs so that a row the call fails to write shows up
        out = {k: torch.full_like(v, float("nan")) for k, v in _outs(w).items()}
        got = windowed_atom_attention(**g.kwargs(), out=out, noalloc=True)
        torch.cuda.synchronize()
        _check(w, got, ref)


def test_noalloc_rejects_sizes_beyond_its_static_buffer():
    w = make_workload("3")  # B=4, A=12288: its workspace exceeds the buffer
    assert workspace_bytes(w.dims, w.style, w.stage, w.dtype) > noalloc_max_bytes()
    g = w.to("cuda")
    with pytest.raises(N.AtomAttnError) as e:
        windowed_atom_attention(**g.kwargs(), noalloc=True)
    assert e.value.code == N.ESCRATCH
