"""Python entry points over libatomattn.so.

``windowed_atom_attention`` mirrors the signature on the page
"windowed_atom_attention -- Local atom attention, encoder pooling and
decoder skip/readout": four dicts plus eps, style, stage and radius, and a
dict result with ``hidden``, ``attention`` and exactly one of
``position_update`` (decoder) / ``token_output`` (encoder).

This layer only marshals arguments: it checks names, shapes and dtypes,
makes non-contiguous inputs contiguous (copies, never in place), allocates
outputs and the workspace with torch, and passes device pointers plus the
current HIP stream to the C ABI. Every step of the block runs in the HIP
kernels; there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import torch

from . import _native as N

_FLOAT_DTYPES = {torch.float32: N.F32, torch.bfloat16: N.BF16}
_STYLES = {"af3": N.AF3, "esmfold2": N.ESMFOLD2}
_STAGES = {"encoder": N.ENCODER, "decoder": N.DECODER}

_ACT_BY_STYLE = {"af3": ("atom", "condition", "pair"),
                 "esmfold2": ("atom", "condition", "rope_cos", "rope_sin")}
_PARAMS_COMMON = ("w_q", "w_k", "w_v", "w_value_gate", "w_attention_out",
                  "w_ff_gate", "w_ff_up", "w_ff_out")
_PARAMS_STYLE = {"af3": ("cond_scale", "w_scale", "b_scale", "w_shift",
                         "w_residual_gate", "b_residual_gate", "b_q",
                         "pair_scale", "w_pair"),
                 "esmfold2": ("w_mod",)}


def _dev_ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _prep(t: torch.Tensor, dtype=None) -> torch.Tensor:
    """Contiguous, 16-byte aligned view or copy (never modifies `t`)."""
    if dtype is not None and t.dtype != dtype:
        raise TypeError("expected dtype %s, got %s" % (dtype, t.dtype))
    if not t.is_contiguous():
        t = t.contiguous()
    if t.data_ptr() % 16 != 0:
        t = t.clone()
    return t


def _mask(t: torch.Tensor) -> torch.Tensor:
    if t.dtype != torch.bool:
        raise TypeError("masks must be torch.bool, got %s" % t.dtype)
    return _prep(t).view(torch.uint8)


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def dims_from(activations, parameters, masks, structure, style, stage) -> Dict[str, int]:
    """B,A,T,K,C,S,H,D,V,M,U read off the supplied shapes (checked)."""
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
        if D_ == 0 or HD % D_ != 0:
            raise ValueError("rope width %d does not divide H*D=%d" % (D_, HD))
        H = HD // D_
        V = 1
    if HD % H != 0:
        raise ValueError("H=%d does not divide H*D=%d" % (H, HD))
    D = HD // H
    U = parameters["w_pool"].shape[-1] if stage == "encoder" else activations["token"].shape[-1]
    d = dict(B=B, A=A, T=T, K=K, C=C, S=S, H=H, D=D, V=V, M=M, U=U)
    if min(B, A, T, K) < 1:
        raise ValueError("zero-size input: B, A, T and K must be >= 1 (got B=%d A=%d T=%d K=%d)"
                         % (B, A, T, K))
    expect = {
        ("activations", "condition"): (B, A, S),
        ("masks", "valid"): (B, A), ("masks", "token_valid"): (B, T),
        ("masks", "window_mask"): (B, A, K),
        ("structure", "atom_to_token"): (B, A), ("structure", "key_index"): (B, A, K),
        ("parameters", "w_q"): (C, HD), ("parameters", "w_k"): (C, HD),
        ("parameters", "w_v"): (C, HD), ("parameters", "w_value_gate"): (C, HD),
        ("parameters", "w_attention_out"): (HD, C),
        ("parameters", "w_ff_gate"): (C, M), ("parameters", "w_ff_up"): (C, M),
        ("parameters", "w_ff_out"): (M, C),
    }
    if style == "af3":
        expect.update({("activations", "pair"): (B, A, K, V),
                       ("parameters", "cond_scale"): (3, S),
                       ("parameters", "w_scale"): (3, S, C),
                       ("parameters", "b_scale"): (3, C),
                       ("parameters", "w_shift"): (3, S, C),
                       ("parameters", "w_residual_gate"): (2, S, C),
                       ("parameters", "b_residual_gate"): (2, C),
                       ("parameters", "b_q"): (HD,),
                       ("parameters", "pair_scale"): (V,),
                       ("parameters", "w_pair"): (V, H)})
    else:
        expect.update({("activations", "rope_cos"): (B, A, D),
                       ("activations", "rope_sin"): (B, A, D),
                       ("parameters", "w_mod"): (S, 6, C)})
    if stage == "encoder":
        expect[("parameters", "w_pool")] = (C, U)
    else:
        expect.update({("activations", "token"): (B, T, U),
                       ("parameters", "w_token"): (U, C),
                       ("parameters", "readout_scale"): (C,),
                       ("parameters", "w_readout"): (C, 3)})
        if style == "esmfold2":
            expect[("parameters", "readout_bias")] = (C,)
    groups = dict(activations=activations, parameters=parameters, masks=masks,
                  structure=structure)
    for (g, name), shape in expect.items():
        if name not in groups[g]:
            raise KeyError("%s is missing %r" % (g, name))
        got = tuple(groups[g][name].shape)
        if got != tuple(shape):
            raise ValueError("%s[%r] has shape %s, expected %s" % (g, name, got, tuple(shape)))
    return d


def workspace_bytes(dims: Dict[str, int], style: str, stage: str, dtype: torch.dtype) -> int:
    nd = N.Dims(**{k: int(v) for k, v in dims.items()})
    out = ctypes.c_size_t(0)
    N.check(N.lib().atom_attn_workspace_bytes(ctypes.byref(nd), _STYLES[style],
                                              _STAGES[stage], _FLOAT_DTYPES[dtype],
                                              ctypes.byref(out)),
            "atom_attn_workspace_bytes")
    return int(out.value)


def packed_bytes(dims: Dict[str, int], style: str, stage: str, dtype: torch.dtype) -> int:
    """Bytes of the packed weight matrices of calls with these sizes."""
    nd = N.Dims(**{k: int(v) for k, v in dims.items()})
    out = ctypes.c_size_t(0)
    N.check(N.lib().atom_attn_packed_bytes(ctypes.byref(nd), _STYLES[style], _STAGES[stage],
                                           _FLOAT_DTYPES[dtype], ctypes.byref(out)),
            "atom_attn_packed_bytes")
    return int(out.value)


def pack_params(parameters: dict, dims: Dict[str, int], style: str, stage: str) -> torch.Tensor:
    """Pack the weight matrices once (atom_attn_pack_params), for block calls
    with the same widths, style, stage and dtype: pass the result as
    `packed=` to windowed_atom_attention. Asynchronous on the current
    stream; keep `parameters` unchanged while the result is in use."""
    dtype = parameters["w_q"].dtype
    dev = parameters["w_q"].device
    if dtype not in _FLOAT_DTYPES or dev.type != "cuda":
        raise ValueError("parameters must be float32/bfloat16 GPU tensors")
    names = list(_PARAMS_COMMON) + list(_PARAMS_STYLE[style])
    names += ["w_pool"] if stage == "encoder" else ["w_token"]
    keep = {k: _prep(parameters[k], dtype) for k in names}
    npar = N.Params(**{k: _dev_ptr(v) for k, v in keep.items()})
    nd = N.Dims(**{k: int(v) for k, v in dims.items()})
    nbytes = packed_bytes(dims, style, stage, dtype)
    out = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        rc = N.lib().atom_attn_pack_params(ctypes.byref(nd), _STYLES[style], _STAGES[stage],
                                           _FLOAT_DTYPES[dtype], ctypes.byref(npar),
                                           out.data_ptr(), nbytes, _stream_handle(dev))
    N.check(rc, "atom_attn_pack_params")
    return out


def window_table(B: int, A: int, K: int, block: int = 32, radius: int = -1,
                 dtype: torch.dtype = torch.int64, device="cuda", out=None) -> torch.Tensor:
    """Windowed key ids [B,A,K] built on the GPU (atom_attn_window_table):
    each block of `block` queries sees K consecutive ids centred on it;
    out-of-range and out-of-radius ids are -1. `out` may supply the
    (contiguous) result tensor."""
    if dtype not in (torch.int64, torch.int32):
        raise TypeError("dtype must be torch.int64 or torch.int32")
    if out is None:
        out = torch.empty((int(B), int(A), int(K)), dtype=dtype, device=device)
    elif (tuple(out.shape) != (int(B), int(A), int(K)) or out.dtype != dtype
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous %s tensor of shape [B,A,K]" % dtype)
    dev = out.device
    with torch.cuda.device(dev):
        rc = N.lib().atom_attn_window_table(int(B), int(A), int(K), int(block), int(radius),
                                            out.element_size(), out.data_ptr(),
                                            _stream_handle(dev))
    N.check(rc, "atom_attn_window_table")
    return out


_S2P_PARAMS = ("weight", "bias", "norm_scale", "norm_bias", "out_weight", "out_bias")


def single_to_pair(activations: dict, parameters: dict, masks: dict, eps: float = 1e-05,
                   output_norm: bool = False, *, out=None):
    """Single-to-pair features on the GPU (atom_attn_single_to_pair), with the
    page's signature: activations {"x" [B,N,C]}, masks {"mask" [B,N] bool},
    parameters {weight [C,2H], bias [2H], norm_scale, norm_bias [C],
    out_weight [2H,D], out_bias [D], and output_scale/output_bias [D] when
    output_norm}. Returns (pair_features [B,N,N,2H], output [B,N,N,D]);
    `out` may supply those two tensors (contiguous, same dtype)."""
    x = activations["x"]
    dtype, dev = x.dtype, x.device
    if dtype not in _FLOAT_DTYPES or dev.type != "cuda":
        raise ValueError("x must be a float32/bfloat16 GPU tensor")
    B, Ntok, C = x.shape
    H2 = parameters["weight"].shape[-1]
    D = parameters["out_weight"].shape[-1]
    names = list(_S2P_PARAMS) + (["output_scale", "output_bias"] if output_norm else [])
    keep = [_prep(x, dtype), _mask(masks["mask"])]
    pp = {k: _prep(parameters[k], dtype) for k in names}
    for k, v in pp.items():
        if v.device != dev:
            raise ValueError("all tensors must share one device")
    nd = N.S2PDims(B=B, N=Ntok, C=C, H=H2 // 2, D=D)
    need = ctypes.c_size_t(0)
    N.check(N.lib().atom_attn_single_to_pair_workspace_bytes(ctypes.byref(nd),
                                                             _FLOAT_DTYPES[dtype],
                                                             ctypes.byref(need)),
            "atom_attn_single_to_pair_workspace_bytes")
    ws = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
    if out is None:
        pf = torch.empty((B, Ntok, Ntok, H2), dtype=dtype, device=dev)
        out = torch.empty((B, Ntok, Ntok, D), dtype=dtype, device=dev)
    else:
        pf, out = out
        for t, shp in ((pf, (B, Ntok, Ntok, H2)), (out, (B, Ntok, Ntok, D))):
            if tuple(t.shape) != shp or t.dtype != dtype or not t.is_contiguous():
                raise ValueError("out tensors must be contiguous %s of shape %s" % (dtype, shp))
    g = lambda k: _dev_ptr(pp.get(k))
    with torch.cuda.device(dev):
        rc = N.lib().atom_attn_single_to_pair(
            ctypes.byref(nd), _FLOAT_DTYPES[dtype], float(eps), 1 if output_norm else 0,
            keep[0].data_ptr(), keep[1].data_ptr(), g("weight"), g("bias"), g("norm_scale"),
            g("norm_bias"), g("out_weight"), g("out_bias"), g("output_scale"),
            g("output_bias"), pf.data_ptr(), out.data_ptr(), ws.data_ptr(), int(need.value),
            _stream_handle(dev))
    N.check(rc, "atom_attn_single_to_pair")
    del keep, pp
    return pf, out


_TIED_PARAMS = ("norm_scale", "norm_bias", "bias_norm_scale", "bias_norm_bias", "w_q", "w_k",
                "w_v", "w_bias", "w_gate", "w_out", "b_out")


def tied_row_attention(activations: dict, parameters: dict, eps: float = 1e-05, *, out=None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Tied pair row attention on the GPU (atom_attn_tied_row_attention),
    with the page's signature: activations {"features" [B,L,L,C],
    "bias_features" [B,L,L,CB]}, parameters {norm_scale, norm_bias [C],
    bias_norm_scale, bias_norm_bias [CB], w_q, w_k, w_v, w_gate [C,H*D],
    w_bias [CB,H], w_out [H*D,C], b_out [C]}. Returns the update [B,L,L,C]
    (no residual added)."""
    f = activations["features"]
    dtype, dev = f.dtype, f.device
    if dtype not in _FLOAT_DTYPES or dev.type != "cuda":
        raise ValueError("features must be a float32/bfloat16 GPU tensor")
    B, L, L2, C = f.shape
    if L2 != L:
        raise ValueError("features must be a square pair grid [B,L,L,C]")
    fb = _prep(activations["bias_features"], dtype)
    CB = fb.shape[-1]
    H = parameters["w_bias"].shape[-1]
    HD = parameters["w_q"].shape[-1]
    keep = [_prep(f, dtype), fb]
    pp = {k: _prep(parameters[k], dtype) for k in _TIED_PARAMS}
    nd = N.TiedDims(B=B, L=L, C=C, CB=CB, H=H, D=HD // H)
    need = ctypes.c_size_t(0)
    N.check(N.lib().atom_attn_tied_row_attention_workspace_bytes(
        ctypes.byref(nd), _FLOAT_DTYPES[dtype], ctypes.byref(need)),
        "atom_attn_tied_row_attention_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need.value:
        raise ValueError("workspace needs %d bytes" % need.value)
    if out is None:
        out = torch.empty((B, L, L, C), dtype=dtype, device=dev)
    elif tuple(out.shape) != (B, L, L, C) or out.dtype != dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous %s tensor [B,L,L,C]" % dtype)
    with torch.cuda.device(dev):
        rc = N.lib().atom_attn_tied_row_attention(
            ctypes.byref(nd), _FLOAT_DTYPES[dtype], float(eps), keep[0].data_ptr(),
            keep[1].data_ptr(), *[pp[k].data_ptr() for k in _TIED_PARAMS], out.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_handle(dev))
    N.check(rc, "atom_attn_tied_row_attention")
    del keep, pp
    return out


def tied_workspace_bytes(B, L, C, CB, H, D, dtype) -> int:
    nd = N.TiedDims(B=B, L=L, C=C, CB=CB, H=H, D=D)
    need = ctypes.c_size_t(0)
    N.check(N.lib().atom_attn_tied_row_attention_workspace_bytes(
        ctypes.byref(nd), _FLOAT_DTYPES[dtype], ctypes.byref(need)),
        "atom_attn_tied_row_attention_workspace_bytes")
    return int(need.value)


def noalloc_max_bytes() -> int:
    """Size of the static per-device scratch of atom_attn_block_noalloc."""
    return int(N.lib().atom_attn_noalloc_max_bytes())


def pair_bias_split(dims: Dict[str, int], style: str, stage: str, dtype: torch.dtype) -> bool:
    """True when a block call with these sizes computes the AF3 pair bias in
    extra workgroups of the projection kernel (on compute units its tiles
    leave idle on the current device) rather than inside the slot kernel."""
    nd = N.Dims(**{k: int(v) for k, v in dims.items()})
    out = ctypes.c_int(0)
    N.check(N.lib().atom_attn_pair_bias_split(ctypes.byref(nd), _STYLES[style],
                                              _STAGES[stage], _FLOAT_DTYPES[dtype],
                                              ctypes.byref(out)),
            "atom_attn_pair_bias_split")
    return bool(out.value)


def _marshal(activations, parameters, masks, structure, style, stage, radius):
    """Checked, contiguous device copies/views of the block's inputs and
    their C structs: (dims, dtype, device, Inputs, Params, keep-alive list)."""
    if style not in _STYLES:
        raise ValueError("style must be 'af3' or 'esmfold2', got %r" % (style,))
    if stage not in _STAGES:
        raise ValueError("stage must be 'encoder' or 'decoder', got %r" % (stage,))
    if isinstance(radius, bool) or int(radius) != radius or radius < -1:
        raise ValueError("radius must be an integer >= -1")
    d = dims_from(activations, parameters, masks, structure, style, stage)
    atom = activations["atom"]
    dtype = atom.dtype
    if dtype not in _FLOAT_DTYPES:
        raise TypeError("float tensors must be float32 or bfloat16, got %s" % dtype)
    dev = atom.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device, got %s" % dev)

    keep = []

    def f(t):
        if t is None:
            return None
        if t.device != dev:
            raise ValueError("all tensors must share one device")
        t = _prep(t, dtype)
        keep.append(t)
        return t

    def ix(t):
        if t.dtype != torch.int64:
            raise TypeError("indices must be int64, got %s" % t.dtype)
        if t.device != dev:
            raise ValueError("all tensors must share one device")
        t = _prep(t)
        keep.append(t)
        return t

    def mk(t):
        if t.device != dev:
            raise ValueError("all tensors must share one device")
        t = _mask(t)
        keep.append(t)
        return t

    acts = {k: f(activations.get(k)) for k in _ACT_BY_STYLE[style]}
    if stage == "decoder":
        acts["token"] = f(activations["token"])
    names = list(_PARAMS_COMMON) + list(_PARAMS_STYLE[style])
    names += ["w_pool"] if stage == "encoder" else ["w_token", "readout_scale", "w_readout"]
    if stage == "decoder" and style == "esmfold2":
        names.append("readout_bias")
    pars = {k: f(parameters[k]) for k in names}

    nin = N.Inputs(
        atom=_dev_ptr(acts.get("atom")), condition=_dev_ptr(acts.get("condition")),
        pair=_dev_ptr(acts.get("pair")), token=_dev_ptr(acts.get("token")),
        rope_cos=_dev_ptr(acts.get("rope_cos")), rope_sin=_dev_ptr(acts.get("rope_sin")),
        valid=_dev_ptr(mk(masks["valid"])),
        token_valid=_dev_ptr(mk(masks["token_valid"])),
        window_mask=_dev_ptr(mk(masks["window_mask"])),
        atom_to_token=_dev_ptr(ix(structure["atom_to_token"])),
        key_index=_dev_ptr(ix(structure["key_index"])))
    npar = N.Params(**{k: _dev_ptr(v) for k, v in pars.items()})
    return d, dtype, dev, nin, npar, keep


def windowed_atom_attention(activations: dict, parameters: dict, masks: dict,
                            structure: dict, eps: float = 1e-05,
                            style: str = "af3", stage: str = "decoder",
                            radius: int = -1, *, workspace: Optional[torch.Tensor] = None,
                            status: Optional[torch.Tensor] = None,
                            out: Optional[Dict[str, torch.Tensor]] = None,
                            noalloc: bool = False,
                            packed: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """One windowed atom-attention block on the GPU.

    Returns {"hidden" [B,A,C], "attention" [B,H,A,K]} plus "token_output"
    [B,T,U] (encoder) or "position_update" [B,A,3] (decoder), in the input
    float dtype (float32 or bfloat16). `workspace` (uint8, at least
    workspace_bytes(...) bytes), `status` (int32 [1]) and preallocated
    `out` tensors are optional; the call is asynchronous on the current
    stream. With `noalloc=True` the call goes to atom_attn_block_noalloc,
    whose scratch is the library's static per-device buffer (no workspace;
    with `out` given and contiguous inputs nothing is allocated). `packed`
    is the result of pack_params(...) for these parameters: the call then
    skips packing the weight matrices."""
    d, dtype, dev, nin, npar, keep = _marshal(activations, parameters, masks, structure, style,
                                              stage, radius)
    if packed is not None:
        need_p = packed_bytes(d, style, stage, dtype)
        if (packed.dtype != torch.uint8 or packed.device != dev or not packed.is_contiguous()
                or packed.numel() < need_p or packed.data_ptr() % 16 != 0):
            raise ValueError("packed must be the uint8 device tensor pack_params returns "
                             "(%d bytes)" % need_p)
        npar.packed = packed.data_ptr()

    B, A, T, K, C, H, U = (d[k] for k in "B A T K C H U".split())
    res = dict(out) if out is not None else {}

    def o(name, shape):
        t = res.get(name)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=dev)
            res[name] = t
        elif tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
            raise ValueError("out[%r] must be a contiguous %s tensor of shape %s" % (name, dtype, shape))
        return t

    nout = N.Outputs(hidden=_dev_ptr(o("hidden", (B, A, C))),
                     attention=_dev_ptr(o("attention", (B, H, A, K))))
    if stage == "encoder":
        nout.token_output = _dev_ptr(o("token_output", (B, T, U)))
    else:
        nout.position_update = _dev_ptr(o("position_update", (B, A, 3)))
    if status is not None:
        if status.dtype != torch.int32 or status.numel() < 1 or status.device != dev:
            raise ValueError("status must be an int32 device tensor with >= 1 element")
        nout.status = status.data_ptr()

    nd = N.Dims(**{k: int(v) for k, v in d.items()})
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc calls take no workspace")
        with torch.cuda.device(dev):
            rc = N.lib().atom_attn_block_noalloc(
                ctypes.byref(nd), _STYLES[style], _STAGES[stage], _FLOAT_DTYPES[dtype],
                ctypes.byref(nin), ctypes.byref(npar), float(eps), int(radius),
                ctypes.byref(nout), _stream_handle(dev))
        N.check(rc, "atom_attn_block_noalloc")
        del keep
        names_out = ["hidden", "attention",
                     "token_output" if stage == "encoder" else "position_update"]
        return {k: res[k] for k in names_out}
    need = workspace_bytes(d, style, stage, dtype)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need or workspace.device != dev:
        raise ValueError("workspace needs %d bytes on %s" % (need, dev))
    fn = N.lib().atom_attn_encoder if stage == "encoder" else N.lib().atom_attn_decoder
    with torch.cuda.device(dev):
        rc = fn(ctypes.byref(nd), _STYLES[style], _FLOAT_DTYPES[dtype],
                ctypes.byref(nin), ctypes.byref(npar), float(eps), int(radius),
                ctypes.byref(nout), workspace.data_ptr(),
                workspace.numel() * workspace.element_size(), _stream_handle(dev))
    N.check(rc, "atom_attn_%s" % stage)
    # Copies made above are freed when `keep` goes away; torch's allocator
    # hands their memory only to later work on this same stream, which runs
    # after the kernels, so no synchronisation is needed.
    del keep
    names_out = ["hidden", "attention", "token_output" if stage == "encoder" else "position_update"]
    return {k: res[k] for k in names_out}


def backward_workspace_bytes(dims: Dict[str, int], style: str, stage: str,
                             dtype: torch.dtype) -> int:
    """Bytes of device workspace one block_backward call needs."""
    nd = N.Dims(**{k: int(v) for k, v in dims.items()})
    need = ctypes.c_size_t(0)
    N.check(N.lib().atom_attn_backward_workspace_bytes(
        ctypes.byref(nd), _STYLES[style], _STAGES[stage], _FLOAT_DTYPES[dtype],
        ctypes.byref(need)), "atom_attn_backward_workspace_bytes")
    return int(need.value)


def block_backward(activations: dict, parameters: dict, masks: dict, structure: dict,
                   grad_outputs: dict, eps: float = 1e-05, style: str = "af3",
                   stage: str = "decoder", radius: int = -1, *,
                   workspace: Optional[torch.Tensor] = None, inputs: Optional[tuple] = None,
                   params: Optional[tuple] = None):
    """Gradients of the block on the GPU (atom_attn_backward).

    grad_outputs: upstream gradients by output name ("hidden", "attention",
    "token_output" / "position_update"; a missing one is zero), any float
    dtype (passed as fp32). Returns (input_grads, param_grads): dicts of
    fp32 tensors for every float input of the style/stage and every
    parameter it reads, or only those named in `inputs` / `params`.
    Asynchronous on the current stream."""
    d, dtype, dev, nin, npar, keep = _marshal(activations, parameters, masks, structure,
                                              style, stage, radius)
    B, A, T, K, C, H, D, U, V = (d[k] for k in "B A T K C H D U V".split())
    up_shapes = {"hidden": (B, A, C), "attention": (B, H, A, K)}
    if stage == "encoder":
        up_shapes["token_output"] = (B, T, U)
    else:
        up_shapes["position_update"] = (B, A, 3)
    gout = N.GradOutputs()
    for name, g in grad_outputs.items():
        if name not in up_shapes:
            raise ValueError("no output %r for stage %r" % (name, stage))
        if g is None:
            continue
        if tuple(g.shape) != up_shapes[name] or g.device != dev:
            raise ValueError("grad_outputs[%r] must have shape %s on %s"
                             % (name, up_shapes[name], dev))
        g = _prep(g.float())
        keep.append(g)
        setattr(gout, name, g.data_ptr())

    in_names = list(_ACT_BY_STYLE[style]) + (["token"] if stage == "decoder" else [])
    par_names = [k for k in N.PARAM_NAMES if k != "packed" and getattr(npar, k)]
    if inputs is not None:
        in_names = [k for k in in_names if k in inputs]
    if params is not None:
        par_names = [k for k in par_names if k in params]
    din = {k: torch.empty(activations[k].shape, dtype=torch.float32, device=dev)
           for k in in_names}
    dpar = {k: torch.empty(parameters[k].shape, dtype=torch.float32, device=dev)
            for k in par_names}
    gin = N.InputGrads(**{k: v.data_ptr() for k, v in din.items()})
    gpar = N.ParamGrads(**{k: v.data_ptr() for k, v in dpar.items()})
    need = backward_workspace_bytes(d, style, stage, dtype)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif (workspace.numel() * workspace.element_size() < need or workspace.device != dev
          or workspace.data_ptr() % 256 != 0):
        raise ValueError("workspace needs %d bytes (256-byte aligned) on %s" % (need, dev))
    nd = N.Dims(**{k: int(v) for k, v in d.items()})
    with torch.cuda.device(dev):
        rc = N.lib().atom_attn_backward(
            ctypes.byref(nd), _STYLES[style], _STAGES[stage], _FLOAT_DTYPES[dtype],
            ctypes.byref(nin), ctypes.byref(npar), float(eps), int(radius),
            ctypes.byref(gout), ctypes.byref(gin), ctypes.byref(gpar), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_handle(dev))
    N.check(rc, "atom_attn_backward")
    del keep
    return din, dpar


def slot_attention_backward(q, k, v, usable, key_index, window_mask, d_o, heads: int,
                            d_attention=None, eps: float = 1e-5, style: str = "af3",
                            radius: int = -1, pair=None, pair_scale=None, w_pair=None):
    """Gradients of the slot-attention step alone (fp32 q, k, v [B,A,H*D];
    AF3 pair [B,A,K,V] with pair_scale [V] and w_pair [V,H] in one float
    dtype). Returns a dict with dq, dk, dv (and d_pair, d_pair_scale,
    d_w_pair for AF3) plus the recomputed attention [B,H,A,K] and o, all
    fp32."""
    q, k, v = (_prep(x.float()) for x in (q, k, v))
    B, A, HD = q.shape
    K = key_index.shape[-1]
    H = int(heads)
    D = HD // H
    dev = q.device
    us = _prep(usable.to(torch.uint8))
    ki = _prep(key_index, torch.int64)
    wm = _mask(window_mask)
    g_o = _prep(d_o.float())
    g_a = _prep(d_attention.float()) if d_attention is not None else None
    keep = [q, k, v, us, ki, wm, g_o, g_a]
    V, dtype = 1, torch.float32
    ptrs = [None, None, None]
    if style == "af3":
        dtype = pair.dtype
        pair, pair_scale, w_pair = (_prep(x, dtype) for x in (pair, pair_scale, w_pair))
        keep += [pair, pair_scale, w_pair]
        V = pair.shape[-1]
        ptrs = [pair.data_ptr(), pair_scale.data_ptr(), w_pair.data_ptr()]
    f32 = dict(dtype=torch.float32, device=dev)
    res = {"attention": torch.empty((B, H, A, K), **f32), "o": torch.empty((B, A, HD), **f32),
           "dq": torch.empty((B, A, HD), **f32), "dk": torch.empty((B, A, HD), **f32),
           "dv": torch.empty((B, A, HD), **f32)}
    if style == "af3":
        res.update(d_pair=torch.empty((B, A, K, V), **f32),
                   d_pair_scale=torch.empty((V,), **f32), d_w_pair=torch.empty((V, H), **f32))
    nd = N.Dims(B=B, A=A, T=1, K=K, C=1, S=1, H=H, D=D, V=V, M=1, U=1)
    need = ctypes.c_size_t(0)
    N.check(N.lib().atom_attn_slot_backward_workspace_bytes(ctypes.byref(nd), _STYLES[style],
                                                            ctypes.byref(need)),
            "atom_attn_slot_backward_workspace_bytes")
    ws = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
    p = lambda name: res[name].data_ptr() if name in res else None
    with torch.cuda.device(dev):
        rc = N.lib().atom_attn_slot_attention_backward(
            ctypes.byref(nd), _STYLES[style], _FLOAT_DTYPES[dtype], float(eps), int(radius),
            us.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), ki.data_ptr(),
            wm.data_ptr(), ptrs[0], ptrs[1], ptrs[2],
            g_a.data_ptr() if g_a is not None else None, g_o.data_ptr(),
            p("attention"), p("o"), p("dq"), p("dk"), p("dv"), p("d_pair"),
            p("d_pair_scale"), p("d_w_pair"), ws.data_ptr(), int(need.value),
            _stream_handle(dev))
    N.check(rc, "atom_attn_slot_attention_backward")
    torch.cuda.current_stream(dev).synchronize()
    del keep
    return res


def masks(masks: dict, structure: dict, T: int, radius: int = -1):
    """usable [B,A] and allowed [B,A,K] (torch.bool) and token_count [B,T]
    (torch.int32, usable atoms per token) computed on the GPU."""
    valid = _mask(masks["valid"])
    tv = _mask(masks["token_valid"])
    wm = _mask(masks["window_mask"])
    a2t = _prep(structure["atom_to_token"], torch.int64)
    ki = _prep(structure["key_index"], torch.int64)
    B, A, K = ki.shape
    dev = ki.device
    usable = torch.empty((B, A), dtype=torch.uint8, device=dev)
    allowed = torch.empty((B, A, K), dtype=torch.uint8, device=dev)
    count = torch.empty((B, int(T)), dtype=torch.int32, device=dev)
    nd = N.Dims(B=B, A=A, T=int(T), K=K, C=1, S=1, H=1, D=1, V=1, M=1, U=1)
    nin = N.Inputs(valid=valid.data_ptr(), token_valid=tv.data_ptr(),
                   window_mask=wm.data_ptr(), atom_to_token=a2t.data_ptr(),
                   key_index=ki.data_ptr())
    with torch.cuda.device(dev):
        rc = N.lib().atom_attn_masks(ctypes.byref(nd), ctypes.byref(nin), int(radius),
                                     usable.data_ptr(), allowed.data_ptr(),
                                     count.data_ptr(), _stream_handle(dev))
    N.check(rc, "atom_attn_masks")
    torch.cuda.current_stream(dev).synchronize()
    return usable.bool(), allowed.bool(), count


def slot_attention(q, k, v, usable, key_index, window_mask, heads: int,
                   eps: float = 1e-5, style: str = "af3", radius: int = -1,
                   pair=None, pair_scale=None, w_pair=None):
    """The slot-attention step alone on supplied q/k/v rows [B,A,H*D]
    (q and k are taken in fp32, v sets the dtype). Returns attention
    [B,H,A,K] and o [B,A,H*D] in v's dtype."""
    dtype = v.dtype
    v = _prep(v, dtype)
    q, k = (_prep(x.float()) for x in (q, k))
    B, A, HD = q.shape
    K = key_index.shape[-1]
    H = int(heads)
    D = HD // H
    us = _prep(usable.to(torch.uint8))
    ki = _prep(key_index, torch.int64)
    wm = _mask(window_mask)
    V = 1
    ptrs = [None, None, None]
    keep = []
    if style == "af3":
        pair, pair_scale, w_pair = (_prep(x, dtype) for x in (pair, pair_scale, w_pair))
        keep += [pair, pair_scale, w_pair]
        V = pair.shape[-1]
        ptrs = [pair.data_ptr(), pair_scale.data_ptr(), w_pair.data_ptr()]
    dev = q.device
    att = torch.empty((B, H, A, K), dtype=dtype, device=dev)
    o = torch.empty((B, A, HD), dtype=dtype, device=dev)
    nd = N.Dims(B=B, A=A, T=1, K=K, C=1, S=1, H=H, D=D, V=V, M=1, U=1)
    need = ctypes.c_size_t(0)
    N.check(N.lib().atom_attn_slot_workspace_bytes(ctypes.byref(nd), _FLOAT_DTYPES[dtype],
                                                   ctypes.byref(need)),
            "atom_attn_slot_workspace_bytes")
    ws = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        rc = N.lib().atom_attn_slot_attention(
            ctypes.byref(nd), _STYLES[style], _FLOAT_DTYPES[dtype], float(eps),
            int(radius), us.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
            ki.data_ptr(), wm.data_ptr(), ptrs[0], ptrs[1], ptrs[2],
            att.data_ptr(), o.data_ptr(), ws.data_ptr(), int(need.value),
            _stream_handle(dev))
    N.check(rc, "atom_attn_slot_attention")
    torch.cuda.current_stream(dev).synchronize()
    return att, o


def profile_enable(on: bool = True) -> None:
    N.check(N.lib().atom_attn_profile_enable(1 if on else 0), "atom_attn_profile_enable")


def profile_read(max_kernels: int = 16) -> Dict[str, tuple]:
    """{kernel name: (total milliseconds, launches)} since the last read."""
    names = (ctypes.c_char_p * max_kernels)()
    ms = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int64 * max_kernels)()
    n = N.lib().atom_attn_profile_read(names, ms, cnt, max_kernels)
    if n < 0:
        N.check(n, "atom_attn_profile_read")
    return {names[i].decode(): (ms[i], int(cnt[i])) for i in range(n)}
