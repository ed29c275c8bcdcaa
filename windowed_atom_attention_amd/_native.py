"""ctypes view of libatomattn.so (include/atom_attn.h). Marshalling only."""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libatomattn.so")

OK, EINVAL, EODD_HEAD, EWORKSPACE, ELAUNCH, EUNSUPPORTED, ESCRATCH = 0, -1, -2, -3, -4, -5, -6
AF3, ESMFOLD2 = 0, 1
F32, BF16 = 0, 1
ENCODER, DECODER = 0, 1

_vp = ctypes.c_void_p


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in "B A T K C S H D V M U".split()]


class Inputs(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("atom", "condition", "pair", "token",
                                   "rope_cos", "rope_sin", "valid",
                                   "token_valid", "window_mask",
                                   "atom_to_token", "key_index")]


PARAM_NAMES = ("cond_scale", "w_scale", "b_scale", "w_shift",
               "w_residual_gate", "b_residual_gate", "w_mod", "w_q", "b_q",
               "w_k", "w_v", "pair_scale", "w_pair", "w_value_gate",
               "w_attention_out", "w_ff_gate", "w_ff_up", "w_ff_out",
               "w_pool", "w_token", "readout_scale", "readout_bias",
               "w_readout", "packed")


class Params(ctypes.Structure):
    _fields_ = [(n, _vp) for n in PARAM_NAMES]


class S2PDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in "B N C H D".split()]


class TiedDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in "B L C CB H D".split()]


class Outputs(ctypes.Structure):
    _fields_ = [("hidden", _vp), ("attention", _vp), ("token_output", _vp),
                ("position_update", _vp), ("status", _vp)]


class GradOutputs(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("hidden", "attention", "token_output", "position_update")]


INPUT_GRAD_NAMES = ("atom", "condition", "pair", "token", "rope_cos", "rope_sin")


class InputGrads(ctypes.Structure):
    _fields_ = [(n, _vp) for n in INPUT_GRAD_NAMES]


class ParamGrads(ctypes.Structure):
    _fields_ = [(n, _vp) for n in PARAM_NAMES if n != "packed"]


EXPORTS = ("atom_attn_workspace_bytes", "atom_attn_encoder",
           "atom_attn_decoder", "atom_attn_masks", "atom_attn_slot_attention",
           "atom_attn_slot_workspace_bytes", "atom_attn_pair_bias_split",
           "atom_attn_error_string", "atom_attn_version",
           "atom_attn_profile_enable", "atom_attn_profile_read",
           "atom_attn_block_noalloc", "atom_attn_noalloc_max_bytes",
           "atom_attn_packed_bytes", "atom_attn_pack_params", "atom_attn_window_table",
           "atom_attn_single_to_pair_workspace_bytes", "atom_attn_single_to_pair",
           "atom_attn_tied_row_attention_workspace_bytes", "atom_attn_tied_row_attention",
           "atom_attn_backward_workspace_bytes", "atom_attn_backward",
           "atom_attn_slot_backward_workspace_bytes", "atom_attn_slot_attention_backward")

_lock = threading.Lock()
_lib = None


class NativeLibraryMissing(ImportError):
    pass


def lib():
    """The loaded library. Raises NativeLibraryMissing if it was not built:
    there is no fallback path."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise NativeLibraryMissing(
                "libatomattn.so is not built (expected at %s); build it with "
                "`python -m windowed_atom_attention_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        i32, i64, dbl, szt = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
        L.atom_attn_workspace_bytes.argtypes = [P(Dims), i32, i32, i32, P(szt)]
        block = [P(Dims), i32, i32, P(Inputs), P(Params), dbl, i64, P(Outputs),
                 _vp, szt, _vp]
        L.atom_attn_encoder.argtypes = block
        L.atom_attn_decoder.argtypes = block
        L.atom_attn_block_noalloc.argtypes = [P(Dims), i32, i32, i32, P(Inputs), P(Params),
                                              dbl, i64, P(Outputs), _vp]
        L.atom_attn_noalloc_max_bytes.argtypes = []
        L.atom_attn_noalloc_max_bytes.restype = szt
        L.atom_attn_packed_bytes.argtypes = [P(Dims), i32, i32, i32, P(szt)]
        L.atom_attn_pack_params.argtypes = [P(Dims), i32, i32, i32, P(Params), _vp, szt, _vp]
        L.atom_attn_window_table.argtypes = [i64, i64, i64, i64, i64, i32, _vp, _vp]
        L.atom_attn_single_to_pair_workspace_bytes.argtypes = [P(S2PDims), i32, P(szt)]
        L.atom_attn_single_to_pair.argtypes = [P(S2PDims), i32, dbl, i32] + [_vp] * 13 + [szt, _vp]
        L.atom_attn_tied_row_attention_workspace_bytes.argtypes = [P(TiedDims), i32, P(szt)]
        L.atom_attn_tied_row_attention.argtypes = [P(TiedDims), i32, dbl] + [_vp] * 15 + [szt, _vp]
        L.atom_attn_masks.argtypes = [P(Dims), P(Inputs), i64, _vp, _vp, _vp, _vp]
        L.atom_attn_slot_attention.argtypes = [P(Dims), i32, i32, dbl, i64, _vp,
                                               _vp, _vp, _vp, _vp, _vp, _vp,
                                               _vp, _vp, _vp, _vp, _vp, szt, _vp]
        L.atom_attn_slot_workspace_bytes.argtypes = [P(Dims), i32, P(szt)]
        L.atom_attn_pair_bias_split.argtypes = [P(Dims), i32, i32, i32, P(i32)]
        L.atom_attn_backward_workspace_bytes.argtypes = [P(Dims), i32, i32, i32, P(szt)]
        L.atom_attn_backward.argtypes = [P(Dims), i32, i32, i32, P(Inputs), P(Params), dbl, i64,
                                         P(GradOutputs), P(InputGrads), P(ParamGrads), _vp,
                                         szt, _vp]
        L.atom_attn_slot_backward_workspace_bytes.argtypes = [P(Dims), i32, P(szt)]
        L.atom_attn_slot_attention_backward.argtypes = [P(Dims), i32, i32, dbl, i64] + \
            [_vp] * 20 + [szt, _vp]
        L.atom_attn_error_string.argtypes = [i32]
        L.atom_attn_error_string.restype = ctypes.c_char_p
        L.atom_attn_version.argtypes = []
        L.atom_attn_profile_enable.argtypes = [i32]
        L.atom_attn_profile_read.argtypes = [P(ctypes.c_char_p), P(dbl), P(i64), i32]
        for name in ("atom_attn_workspace_bytes", "atom_attn_encoder",
                     "atom_attn_decoder", "atom_attn_masks",
                     "atom_attn_slot_attention", "atom_attn_slot_workspace_bytes",
                     "atom_attn_pair_bias_split", "atom_attn_version",
                     "atom_attn_block_noalloc", "atom_attn_packed_bytes",
                     "atom_attn_pack_params", "atom_attn_window_table",
                     "atom_attn_single_to_pair_workspace_bytes", "atom_attn_single_to_pair",
                     "atom_attn_tied_row_attention_workspace_bytes",
                     "atom_attn_tied_row_attention",
                     "atom_attn_backward_workspace_bytes", "atom_attn_backward",
                     "atom_attn_slot_backward_workspace_bytes",
                     "atom_attn_slot_attention_backward",
                     "atom_attn_profile_enable", "atom_attn_profile_read"):
            getattr(L, name).restype = i32
        _lib = L
        return L


def error_string(code: int) -> str:
    return lib().atom_attn_error_string(int(code)).decode()


class AtomAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed with status %d: %s" % (where, code, error_string(code)))


def check(code: int, where: str) -> None:
    if code != OK:
        raise AtomAttnError(code, where)
