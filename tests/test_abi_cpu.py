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
    assert lib.atom_attn_version() == 6


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


def test_shapes_whose_32bit_value_offsets_would_overflow_are_rejected():
    """The slot kernel reads one head's transposed value rows through a
    32-bit byte offset of up to D * (A rounded up to 8, + 32) * sizeof(dtype):
    shapes where that reaches 2^31 are outside the supported set, for the
    block and for the standalone slot step."""
    big = dict(H=1, D=128, K=1, T=8)
    # fp32: 128 * 4 * pitch >= 2^31 once pitch >= 4194304
    assert _ws(_dims(A=4_194_304 - 40, **big))[0] == N.OK
    assert _ws(_dims(A=4_194_304, **big))[0] == N.EUNSUPPORTED
    # bf16 halves the bytes per value
    assert _ws(_dims(A=4_194_304, **big), dtype=N.BF16)[0] == N.OK
    assert _ws(_dims(A=8_388_608, **big), dtype=N.BF16)[0] == N.EUNSUPPORTED
    lib = N.lib()
    fake = 4096  # aligned, never dereferenced: rejected before any launch
    for A, dt, rc in ((4_194_304, N.F32, N.EUNSUPPORTED), (8_388_608, N.BF16, N.EUNSUPPORTED)):
        nd = N.Dims(**_dims(A=A, **big))
        got = lib.atom_attn_slot_attention(ctypes.byref(nd), N.ESMFOLD2, dt, 1e-5, -1,
                                           fake, fake, fake, fake, fake, fake, None, None,
                                           None, fake, fake, fake, 1 << 40, None)
        assert got == rc, (A, dt, got)


def test_pack_params_status_codes():
    lib = N.lib()
    nd = N.Dims(**_dims())
    n = ctypes.c_size_t(0)
    assert lib.atom_attn_packed_bytes(ctypes.byref(nd), N.AF3, N.ENCODER, N.F32,
                                      ctypes.byref(n)) == N.OK
    # both operand layouts of every matrix: 2 * (8 AF3 conditioning matrices
    # [S,C] + 4 [C,HD] + [HD,C] + 2 [C,M] + [M,C] + w_pool [C,U]) * 4 bytes
    d = _dims()
    C, S, HD, M, U = d["C"], d["S"], d["H"] * d["D"], d["M"], d["U"]
    elems = 8 * S * C + 4 * C * HD + HD * C + 2 * C * M + M * C + C * U
    assert n.value == 2 * elems * 4
    assert lib.atom_attn_packed_bytes(ctypes.byref(nd), N.AF3, N.ENCODER, 9,
                                      ctypes.byref(n)) == N.EINVAL
    fake = 4096  # never dereferenced: rejected on the host
    par = N.Params()
    assert lib.atom_attn_pack_params(ctypes.byref(nd), N.AF3, N.ENCODER, N.F32,
                                     ctypes.byref(par), fake, 1 << 30, None) == N.EINVAL
    full = N.Params(**{k: fake for k in N.PARAM_NAMES if k != "packed"})
    assert lib.atom_attn_pack_params(ctypes.byref(nd), N.AF3, N.ENCODER, N.F32,
                                     ctypes.byref(full), None, 1 << 30, None) == N.EWORKSPACE
    assert lib.atom_attn_pack_params(ctypes.byref(nd), N.AF3, N.ENCODER, N.F32,
                                     ctypes.byref(full), fake, 16, None) == N.EWORKSPACE
    # a misaligned prepacked buffer is rejected by the block call
    nin = N.Inputs(**{k: fake for k, _ in N.Inputs._fields_})
    nout = N.Outputs(hidden=fake, attention=fake, token_output=fake)
    full.packed = fake + 8
    assert lib.atom_attn_encoder(ctypes.byref(nd), N.AF3, N.F32, ctypes.byref(nin),
                                 ctypes.byref(full), 1e-5, -1, ctypes.byref(nout), fake,
                                 1 << 40, None) == N.EINVAL


def test_window_table_status_codes():
    lib = N.lib()
    fake = 4096  # never dereferenced: rejected on the host
    assert lib.atom_attn_window_table(1, 10, 4, 2, -1, 8, None, None) == N.EINVAL
    assert lib.atom_attn_window_table(0, 10, 4, 2, -1, 8, fake, None) == N.EINVAL
    assert lib.atom_attn_window_table(1, 10, 4, 0, -1, 8, fake, None) == N.EINVAL
    assert lib.atom_attn_window_table(1, 10, 4, 2, -2, 8, fake, None) == N.EINVAL
    assert lib.atom_attn_window_table(1, 10, 4, 2, -1, 2, fake, None) == N.EINVAL
    assert lib.atom_attn_window_table(1, 1 << 31, 4, 2, -1, 8, fake, None) == N.EUNSUPPORTED
    assert lib.atom_attn_window_table(1 << 12, 1 << 12, 1 << 8, 32, -1, 8, fake,
                                      None) == N.EUNSUPPORTED


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
    assert lib.atom_attn_masks(ctypes.byref(nd), None, -1, None, None, None, None) == N.EINVAL
    # inputs present but no output requested
    fake = 4096  # never dereferenced: the call is rejected on the host
    nin_m = N.Inputs(valid=fake, token_valid=fake, window_mask=fake, atom_to_token=fake,
                     key_index=fake)
    assert lib.atom_attn_masks(ctypes.byref(nd), ctypes.byref(nin_m), -1, None, None, None,
                               None) == N.EINVAL
    assert lib.atom_attn_masks(ctypes.byref(nd), ctypes.byref(nin_m), -2, fake, fake, fake,
                               None) == N.EINVAL
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
    # zero-size inputs are rejected before anything else happens
    empty = make_workload("0")
    empty.structure["key_index"] = empty.structure["key_index"][..., :0]
    empty.masks["window_mask"] = empty.masks["window_mask"][..., :0]
    empty.activations["pair"] = empty.activations["pair"][:, :, :0]
    with pytest.raises(ValueError, match="zero-size"):
        windowed_atom_attention(**empty.kwargs())


def _bws(d, style=N.AF3, stage=N.ENCODER, dtype=N.F32):
    nd = N.Dims(**d)
    out = ctypes.c_size_t(0)
    rc = N.lib().atom_attn_backward_workspace_bytes(ctypes.byref(nd), style, stage, dtype,
                                                    ctypes.byref(out))
    return rc, out.value


def test_backward_workspace_query_status_codes():
    rc, n = _bws(_dims())
    assert rc == N.OK and n > 0
    assert _bws(_dims(A=0))[0] == N.EINVAL
    assert _bws(_dims(), style=5)[0] == N.EINVAL
    assert _bws(_dims(), stage=2)[0] == N.EINVAL
    assert _bws(_dims(), dtype=9)[0] == N.EINVAL
    assert _bws(_dims(H=4, D=7), style=N.ESMFOLD2)[0] == N.EODD_HEAD
    assert _bws(_dims(D=128, H=2))[0] == N.EUNSUPPORTED     # head width outside 8..64
    assert _bws(_dims(D=12))[0] == N.EUNSUPPORTED
    assert _bws(_dims(K=513))[0] == N.EUNSUPPORTED
    assert _bws(_dims(H=5, D=16))[0] == N.EUNSUPPORTED      # AF3 pair gradients: H <= 4
    assert _bws(_dims(H=5, D=16), style=N.ESMFOLD2)[0] == N.OK
    assert _bws(_dims(V=17))[0] == N.EUNSUPPORTED
    assert _bws(_dims(V=17), style=N.ESMFOLD2)[0] == N.OK   # no pair there
    # rows x widest intermediate (6C) above 2^34 elements
    assert _bws(_dims(A=1 << 21, C=4096, K=8))[0] == N.EUNSUPPORTED
    assert _bws(_dims(A=1 << 18, C=4096, K=8))[0] == N.OK
    # dense widths need not be multiples of 32 here
    assert _bws(_dims(C=48, S=40, M=72, U=20))[0] == N.OK
    # decoder keeps the token projection and its reverse index
    assert _bws(_dims(), stage=N.DECODER)[1] > 0
    for name in ("1", "3", "4a", "4b"):
        w = make_workload(name, A=64)
        st = N.AF3 if w.style == "af3" else N.ESMFOLD2
        sg = N.ENCODER if w.stage == "encoder" else N.DECODER
        assert _bws(w.dims, st, sg, N.BF16)[0] == N.OK


def test_backward_rejects_bad_arguments_before_any_launch():
    lib = N.lib()
    fake = 4096  # never dereferenced: every case fails its checks first
    nd = N.Dims(**_dims())
    ins = N.Inputs()
    par = N.Params()
    gout = N.GradOutputs()
    # missing inputs / parameters
    rc = lib.atom_attn_backward(ctypes.byref(nd), N.AF3, N.ENCODER, N.F32, ctypes.byref(ins),
                                ctypes.byref(par), 1e-5, -1, ctypes.byref(gout), None, None,
                                fake, 1 << 40, None)
    assert rc == N.EINVAL
    for name in N.Inputs._fields_:
        setattr(ins, name[0], fake)
    for name in N.Params._fields_:
        if name[0] != "packed":
            setattr(par, name[0], fake)
    for eps in (0.0, -1.0, float("nan"), float("inf")):
        rc = lib.atom_attn_backward(ctypes.byref(nd), N.AF3, N.ENCODER, N.F32,
                                    ctypes.byref(ins), ctypes.byref(par), eps, -1,
                                    ctypes.byref(gout), None, None, fake, 1 << 40, None)
        assert rc == N.EINVAL, eps
    rc = lib.atom_attn_backward(ctypes.byref(nd), N.AF3, N.ENCODER, N.F32, ctypes.byref(ins),
                                ctypes.byref(par), 1e-5, -2, ctypes.byref(gout), None, None,
                                fake, 1 << 40, None)
    assert rc == N.EINVAL
    # workspace missing, misaligned or short
    for ws, nbytes in ((None, 1 << 40), (fake + 16, 1 << 40), (fake, 16)):
        rc = lib.atom_attn_backward(ctypes.byref(nd), N.AF3, N.ENCODER, N.F32,
                                    ctypes.byref(ins), ctypes.byref(par), 1e-5, -1,
                                    ctypes.byref(gout), None, None, ws, nbytes, None)
        assert rc == N.EWORKSPACE, (ws, nbytes)
    # the slot step: NULL gradient buffers, unsupported head width
    out = ctypes.c_size_t(0)
    assert lib.atom_attn_slot_backward_workspace_bytes(ctypes.byref(nd), N.AF3,
                                                       ctypes.byref(out)) == N.OK
    # usable, q, k, v, key_index, window_mask; pair, pair_scale, w_pair;
    # d_attention, d_o; attention, o; dq (NULL), dk, dv; d_pair, d_pair_scale,
    # d_w_pair; workspace, bytes, stream
    args = [fake] * 6 + [None, None, None, fake, fake, None, None, None, fake, fake, None,
                         None, None, fake, 1 << 40, None]
    rc = lib.atom_attn_slot_attention_backward(ctypes.byref(nd), N.ESMFOLD2, N.F32, 1e-5, -1,
                                               *args)
    assert rc == N.EINVAL
    rc = lib.atom_attn_slot_attention_backward(ctypes.byref(nd), N.AF3, N.F32, 1e-5, -1,
                                               *args)
    assert rc == N.EINVAL                                    # AF3 needs the pair inputs
    bad = N.Dims(**_dims(D=128))
    rc = lib.atom_attn_slot_attention_backward(ctypes.byref(bad), N.ESMFOLD2, N.F32, 1e-5, -1,
                                               *args)
    assert rc == N.EUNSUPPORTED
