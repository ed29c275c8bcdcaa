"""Plain fp64 CPU oracle of the windowed atom-attention block (ctypes wrapper).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
CPU-baseline leg of ``bench.py`` import this package; the product library
never does, and this package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, fp64, straight loops). This
wrapper only marshals arrays: every float input is upcast exactly to float64
(fp32 and bf16 values are representable in fp64), index arrays become int64
and masks uint8.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

AF3, ESMFOLD2 = 0, 1
ENCODER, DECODER = 0, 1
STYLES = {"af3": AF3, "esmfold2": ESMFOLD2}
STAGES = {"encoder": ENCODER, "decoder": DECODER}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA
    contraction, so every sum is the plain one)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in "B A T K C S H D V M U".split()]


_DP = ctypes.POINTER(ctypes.c_double)
_U8P = ctypes.POINTER(ctypes.c_uint8)
_I64P = ctypes.POINTER(ctypes.c_int64)


class _Inputs(ctypes.Structure):
    _fields_ = [("atom", _DP), ("condition", _DP), ("pair", _DP),
                ("token", _DP), ("rope_cos", _DP), ("rope_sin", _DP),
                ("valid", _U8P), ("token_valid", _U8P), ("window_mask", _U8P),
                ("atom_to_token", _I64P), ("key_index", _I64P)]


_PARAM_NAMES = ["cond_scale", "w_scale", "b_scale", "w_shift",
                "w_residual_gate", "b_residual_gate", "w_mod", "w_q", "b_q",
                "w_k", "w_v", "pair_scale", "w_pair", "w_value_gate",
                "w_attention_out", "w_ff_gate", "w_ff_up", "w_ff_out",
                "w_pool", "w_token", "readout_scale", "readout_bias",
                "w_readout"]


class _Params(ctypes.Structure):
    _fields_ = [(n, _DP) for n in _PARAM_NAMES]


class _Outputs(ctypes.Structure):
    _fields_ = [("hidden", _DP), ("attention", _DP), ("token_output", _DP),
                ("position_update", _DP), ("usable", _U8P), ("allowed", _U8P),
                ("x0", _DP), ("q_in", _DP), ("kv_in", _DP), ("q", _DP), ("k", _DP),
                ("v", _DP), ("g", _DP), ("o", _DP), ("x1", _DP),
                ("done_atom", _U8P), ("done_token", _U8P)]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            stale = (not os.path.exists(_LIB_PATH) or
                     os.path.getmtime(_LIB_PATH) < max(
                         os.path.getmtime(_SRC),
                         os.path.getmtime(os.path.join(_HERE, "oracle.h"))))
            if stale:
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            lib.orc_block.restype = ctypes.c_int
            lib.orc_block.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int,
                                      ctypes.c_int, ctypes.c_double,
                                      ctypes.c_int64, ctypes.POINTER(_Inputs),
                                      ctypes.POINTER(_Params), _U8P,
                                      ctypes.POINTER(_Outputs), ctypes.c_int]
            lib.orc_slot_attention.restype = ctypes.c_int
            lib.orc_slot_attention.argtypes = [
                ctypes.POINTER(_Dims), ctypes.c_int, ctypes.c_double,
                ctypes.c_int64, _U8P, _DP, _DP, _DP, _I64P, _U8P, _DP, _DP,
                _DP, _DP, _DP, _U8P, ctypes.c_int]
            lib.orc_threads.restype = ctypes.c_int
            lib.orc_threads.argtypes = [ctypes.c_int]
            _lib = lib
    return _lib


def _np(x, dtype):
    """Host numpy copy of a tensor/array, upcast exactly."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            t = x.detach().to("cpu")
            if dtype == np.float64:
                t = t.to(torch.float64)
            elif dtype == np.int64:
                t = t.to(torch.int64)
            elif dtype == np.uint8:
                t = t.to(torch.uint8)
            return np.ascontiguousarray(t.numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x).astype(dtype))


def _ptr(arr, ctype):
    if arr is None:
        return ctypes.cast(None, ctypes.POINTER(ctype))
    return arr.ctypes.data_as(ctypes.POINTER(ctype))


def threads(nthreads: int = 0) -> int:
    """Threads an oracle call with this `nthreads` argument uses."""
    return int(_load().orc_threads(int(nthreads)))


def dims_of(activations, parameters, masks, structure, style, stage):
    """Read B,A,T,K,C,S,H,D,V,M,U off the supplied shapes."""
    B, A, C = activations["atom"].shape
    S = activations["condition"].shape[-1]
    T = masks["token_valid"].shape[-1]
    K = structure["key_index"].shape[-1]
    HD = parameters["w_q"].shape[-1]
    M = parameters["w_ff_gate"].shape[-1]
    if style == "af3":
        H = parameters["w_pair"].shape[-1]
        V = activations["pair"].shape[-1]
    else:
        D_ = activations["rope_cos"].shape[-1]
        H = HD // D_
        V = 1
    D = HD // H
    if stage == "encoder":
        U = parameters["w_pool"].shape[-1]
    else:
        U = activations["token"].shape[-1]
    return dict(B=B, A=A, T=T, K=K, C=C, S=S, H=H, D=D, V=V, M=M, U=U)


def block(activations, parameters, masks, structure, eps=1e-5, style="af3",
          stage="decoder", radius=-1, select=None, intermediates=False,
          nthreads=0, dims=None):
    """Run the whole block in fp64. Returns a dict of float64/uint8 arrays:
    hidden, attention and position_update (decoder) or token_output
    (encoder); with intermediates=True also usable, allowed, x0, q_in, kv_in,
    q, k, v, g, o, x1; with `select` also done_atom/done_token."""
    lib = _load()
    d = dims or dims_of(activations, parameters, masks, structure, style, stage)
    dd = _Dims(**{k: int(v) for k, v in d.items()})
    B, A, T, K, C = d["B"], d["A"], d["T"], d["K"], d["C"]
    H, D, U = d["H"], d["D"], d["U"]
    keep = []

    def f(x):
        a = _np(x, np.float64)
        keep.append(a)
        return a

    ins = dict(atom=f(activations.get("atom")),
               condition=f(activations.get("condition")),
               pair=f(activations.get("pair")) if style == "af3" else None,
               token=f(activations.get("token")) if stage == "decoder" else None,
               rope_cos=f(activations.get("rope_cos")) if style == "esmfold2" else None,
               rope_sin=f(activations.get("rope_sin")) if style == "esmfold2" else None)
    valid = _np(masks["valid"], np.uint8)
    token_valid = _np(masks["token_valid"], np.uint8)
    window_mask = _np(masks["window_mask"], np.uint8)
    a2t = _np(structure["atom_to_token"], np.int64)
    key_index = _np(structure["key_index"], np.int64)
    keep += [valid, token_valid, window_mask, a2t, key_index]
    cin = _Inputs(atom=_ptr(ins["atom"], ctypes.c_double),
                  condition=_ptr(ins["condition"], ctypes.c_double),
                  pair=_ptr(ins["pair"], ctypes.c_double),
                  token=_ptr(ins["token"], ctypes.c_double),
                  rope_cos=_ptr(ins["rope_cos"], ctypes.c_double),
                  rope_sin=_ptr(ins["rope_sin"], ctypes.c_double),
                  valid=_ptr(valid, ctypes.c_uint8),
                  token_valid=_ptr(token_valid, ctypes.c_uint8),
                  window_mask=_ptr(window_mask, ctypes.c_uint8),
                  atom_to_token=_ptr(a2t, ctypes.c_int64),
                  key_index=_ptr(key_index, ctypes.c_int64))
    pv = {}
    for name in _PARAM_NAMES:
        x = parameters.get(name)
        pv[name] = _ptr(f(x), ctypes.c_double) if x is not None else _ptr(None, ctypes.c_double)
    cpar = _Params(**pv)

    res = {}

    def o(name, shape, dtype=np.float64, fill=np.nan):
        a = np.full(shape, fill, dtype=dtype)
        res[name] = a
        return _ptr(a, ctypes.c_double if dtype == np.float64 else ctypes.c_uint8)

    N = B * A
    HD = H * D
    outs = dict(hidden=o("hidden", (B, A, C)),
                attention=o("attention", (B, H, A, K)))
    if stage == "encoder":
        outs["token_output"] = o("token_output", (B, T, U))
    else:
        outs["position_update"] = o("position_update", (B, A, 3))
    if intermediates:
        outs.update(usable=o("usable", (B, A), np.uint8, 0),
                    allowed=o("allowed", (B, A, K), np.uint8, 0),
                    x0=o("x0", (B, A, C)),
                    q_in=o("q_in", (B, A, C)), kv_in=o("kv_in", (B, A, C)),
                    q=o("q", (B, A, HD)), k=o("k", (B, A, HD)),
                    v=o("v", (B, A, HD)), g=o("g", (B, A, HD)),
                    o=o("o", (B, A, HD)), x1=o("x1", (B, A, C)))
    sel = None
    if select is not None:
        sel = _np(select, np.uint8).reshape(N)
        keep.append(sel)
        outs.update(done_atom=o("done_atom", (B, A), np.uint8, 0),
                    done_token=o("done_token", (B, T), np.uint8, 0))
    cout = _Outputs(**outs)
    rc = lib.orc_block(ctypes.byref(dd), STYLES[style], STAGES[stage],
                       float(eps), int(radius), ctypes.byref(cin),
                       ctypes.byref(cpar), _ptr(sel, ctypes.c_uint8),
                       ctypes.byref(cout), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return res


def slot_attention(q, k, v, usable, key_index, window_mask, eps=1e-5,
                   style="af3", radius=-1, pair=None, pair_scale=None,
                   w_pair=None, heads=1, nthreads=0):
    """Slot-attention step alone from per-atom Q/K/V rows [B,A,H*D].
    Returns attention [B,H,A,K], o [B,A,H*D], allowed [B,A,K]."""
    lib = _load()
    qn, kn, vn = (_np(x, np.float64) for x in (q, k, v))
    B, A, HD = qn.shape
    H = int(heads)
    K = _np(key_index, np.int64).shape[-1]
    V = _np(pair, np.float64).shape[-1] if pair is not None else 1
    dd = _Dims(B=B, A=A, T=1, K=K, C=1, S=1, H=H, D=HD // H, V=V, M=1, U=1)
    us = _np(usable, np.uint8)
    ki = _np(key_index, np.int64)
    wm = _np(window_mask, np.uint8)
    pr = _np(pair, np.float64) if pair is not None else None
    ps = _np(pair_scale, np.float64) if pair_scale is not None else None
    wp = _np(w_pair, np.float64) if w_pair is not None else None
    att = np.full((B, H, A, K), np.nan)
    ob = np.full((B, A, HD), np.nan)
    al = np.zeros((B, A, K), np.uint8)
    rc = lib.orc_slot_attention(
        ctypes.byref(dd), STYLES[style], float(eps), int(radius),
        _ptr(us, ctypes.c_uint8), _ptr(qn, ctypes.c_double),
        _ptr(kn, ctypes.c_double), _ptr(vn, ctypes.c_double),
        _ptr(ki, ctypes.c_int64), _ptr(wm, ctypes.c_uint8),
        _ptr(pr, ctypes.c_double), _ptr(ps, ctypes.c_double),
        _ptr(wp, ctypes.c_double), _ptr(att, ctypes.c_double),
        _ptr(ob, ctypes.c_double), _ptr(al, ctypes.c_uint8), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return {"attention": att, "o": ob, "allowed": al}
