"""Host-side checks of libatomattn.so that need no GPU: the library loads,
exports every entry point include/atom_attn.h declares, and rejects bad
arguments with the documented status codes before enqueuing anything."""
import ctypes
import os
import re

import pytest
import torch

from windowed_atom_attention_amd import _native as N
from windowed_atom_attention_amd import workspace_bytes
from windowed_atom_attention_amd.workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "atom_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(atom_attn_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = N.lib()
    names = _declared()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(N.EXPORTS)
    assert lib.atom_attn_version() == 3


def test_pair_bias_split_query():
    # without a GPU the library assumes 256 compute units (MI355X)
    from windowed_atom_attention_amd import pair_bias_split
    w1 = make_workload("1")     # 144 tiles: 112 idle units host the bias
    assert pair_bias_split(w1.dims, "af3", "encoder", torch.float32)
    w4 = make_workload("4a", A=24576)  # 768 tiles: every unit busy
    assert not pair_bias_split(w4.dims, "af3", "encoder", torch.bfloat16)
    assert not pair_bias_split(make_workload("4b", A=256).dims, "esmfold2", "encoder",
                               torch.bfloat16)
    d = _dims(V=32)             # bf16 rows wider than 16 channels stay fused
    assert not pair_bias_split(d, "af3", "encoder", torch.bfloat16)
    assert pair_bias_split(_dims(), "af3", "encoder", torch.bfloat16)


def test_error_strings():
    for code in (N.OK, N.EINVAL, N.EODD_HEAD, N.EWORKSPACE, N.ELAUNCH, N.EUNSUPPORTED, 7):
        s = N.error_string(code)
        assert isinstance(s, str) and s


def _dims(**kw):
    d = dict(B=1, A=64, T=8, K=16, C=32, S=32, H=2, D=16, V=8, M=64, U=32)
    d.update(kw)
    return d


def _ws(d, style=N.AF3, stage=N.ENCODER, dtype=N.F32):
    nd = N.Dims(**d)
    out = ctypes.c_size_t(0)
    rc = N.lib().atom_attn_workspace_bytes(ctypes.byref(nd), style, stage, dtype,
                                           ctypes.byref(out))
    return rc, out.value


def test_workspace_query_status_codes():
    rc, n = _ws(_dims())
    assert rc == N.OK and n > 0
    assert _ws(_dims(A=0))[0] == N.EINVAL
    assert _ws(_dims(), style=5)[0] == N.EINVAL
    assert _ws(_dims(), stage=2)[0] == N.EINVAL
    assert _ws(_dims(), dtype=9)[0] == N.EINVAL
    assert _ws(_dims(H=4, D=7), style=N.ESMFOLD2)[0] == N.EODD_HEAD
    assert _ws(_dims(C=48))[0] == N.EUNSUPPORTED
    assert _ws(_dims(K=1000))[0] == N.EUNSUPPORTED
    assert _ws(_dims(K=300))[0] == N.EUNSUPPORTED
    assert _ws(_dims(V=32))[0] == N.EUNSUPPORTED            # fp32 pair row > 64 B
    assert _ws(_dims(V=32), dtype=N.BF16)[0] == N.OK
    assert _ws(_dims(V=3))[0] == N.EUNSUPPORTED
    assert _ws(_dims(V=3), style=N.ESMFOLD2)[0] == N.OK  # V unused there
    # decoder adds the fp32 token projection
    assert _ws(_dims(), stage=N.DECODER)[1] > _ws(_dims())[1]


def test_workspace_sizes_of_all_workloads():
    for name in ("0", "1", "2", "3", "4a", "4b"):
        w = make_workload(name, A=64 if name != "0" else None)
        assert workspace_bytes(w.dims, w.style, w.stage, w.dtype) > 0


def test_block_rejects_bad_arguments_before_any_launch():
    lib = N.lib()
    nd = N.Dims(**_dims())
    nin, npar, nout = N.Inputs(), N.Params(), N.Outputs()
    for fn in (lib.atom_attn_encoder, lib.atom_attn_decoder):
        # NULL pointers
        assert fn(ctypes.byref(nd), N.AF3, N.F32, ctypes.byref(nin), ctypes.byref(npar),
                  1e-5, -1, ctypes.byref(nout), None, 0, None) == N.EINVAL
        # eps <= 0 / not finite, radius < -1
        for eps, radius in ((0.0, -1), (-1.0, -1), (float("nan"), -1),
                            (float("inf"), -1), (1e-5, -2)):
            assert fn(ctypes.byref(nd), N.AF3, N.F32, ctypes.byref(nin),
                      ctypes.byref(npar), eps, radius, ctypes.byref(nout), None,
                      0, None) == N.EINVAL
        assert fn(None, N.AF3, N.F32, None, None, 1e-5, -1, None, None, 0, None) == N.EINVAL
    assert lib.atom_attn_masks(ctypes.byref(nd), None, -1, None, None, None) == N.EINVAL
    assert lib.atom_attn_slot_attention(ctypes.byref(nd), N.AF3, N.F32, 1e-5, -1,
                                        None, None, None, None, None, None, None,
                                        None, None, None, None, None, 0, None) == N.EINVAL


def test_python_binding_argument_checks():
    from windowed_atom_attention_amd import windowed_atom_attention
    w = make_workload("0")
    with pytest.raises(ValueError):
        windowed_atom_attention(**dict(w.kwargs(), style="af2"))
    with pytest.raises(ValueError):
        windowed_atom_attention(**dict(w.kwargs(), stage="middle"))
    with pytest.raises(ValueError):
        windowed_atom_attention(**dict(w.kwargs(), radius=-3))
    with pytest.raises(ValueError):  # CPU tensors: the product path is GPU-only
        windowed_atom_attention(**w.kwargs())
    bad = make_workload("0")
    bad.structure["key_index"] = bad.structure["key_index"][..., :5]
    with pytest.raises(ValueError):
        windowed_atom_attention(**bad.kwargs())
