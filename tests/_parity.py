"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (floating point), rtol = 1e-4 for fp32 storage, 2e-2 for bf16
storage with fp32 arithmetic:
* attention weights: |gpu - oracle| <= rtol * |oracle| + 1e-30 elementwise.
  The weights are non-negative softmax terms whose relative error is the
  logit error plus one storage rounding, so no tensor-wide floor is needed
  (the 1e-30 only admits results that underflow to subnormals);
* outputs formed by sums with cancellation (hidden, o, token_output,
  position_update): |gpu - oracle| <= rtol * (|oracle| + rms(oracle)), rms
  over the whole compared tensor, so that an entry that cancels to near
  zero is judged on the scale of its tensor.
Masks, indices and every exact-zero the pages require are compared
bit-exactly."""
import numpy as np
import torch

import oracle
from windowed_atom_attention_amd import windowed_atom_attention

RTOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def np64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def assert_close(name, got, ref, rtol, where=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if where is not None:
        got, ref = got[where], ref[where]
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if ref.size == 0:
        return
    assert np.all(np.isfinite(got)), "%s: non-finite GPU values" % name
    rms = float(np.sqrt(np.mean(ref * ref)))
    tol = rtol * (np.abs(ref) + rms)
    err = np.abs(got - ref)
    bad = err > tol
    print("%s: max err/tol %.3g (rtol=%g, rms floor %.3g)" % (
        name, float(np.max(err / np.maximum(tol, 1e-300))), rtol, rms))
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(tol, 1e-300)), err.shape)
        raise AssertionError(
            "%s: %d/%d elements out of tolerance (rtol=%g, rms=%.3g); worst at %s: "
            "gpu=%.8g oracle=%.8g" % (name, int(bad.sum()), bad.size, rtol, rms,
                                     tuple(int(x) for x in i), got[i], ref[i]))


def assert_close_rel(name, got, ref, rtol, where=None, floor=1e-30):
    """Elementwise relative check for non-negative outputs (attention)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if where is not None:
        got, ref = got[where], ref[where]
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if ref.size == 0:
        return
    assert np.all(np.isfinite(got)), "%s: non-finite GPU values" % name
    tol = rtol * np.abs(ref) + floor
    err = np.abs(got - ref)
    bad = err > tol
    worst = float(np.max(err / tol))
    print("%s: max err/tol %.3g (elementwise relative, rtol=%g)" % (name, worst, rtol))
    if bad.any():
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(
            "%s: %d/%d elements out of tolerance (rtol=%g, elementwise relative); "
            "worst at %s: gpu=%.8g oracle=%.8g" % (name, int(bad.sum()), bad.size, rtol,
                                                  tuple(int(x) for x in i), got[i], ref[i]))


def run_gpu(w, **kw):
    g = w.to("cuda")
    out = windowed_atom_attention(**g.kwargs(), **kw)
    torch.cuda.synchronize()
    return out


def exact_zero_checks(w, gpu, usable, allowed):
    """Zeros the pages fix: attention off the allowed slots, hidden (and
    position_update) of unusable atoms, token_output of empty tokens."""
    att = np64(gpu["attention"])
    al = np.asarray(allowed, bool)  # [B,A,K]
    assert np.all(att[np.broadcast_to(~al[:, None], att.shape)] == 0.0)
    us = np.asarray(usable, bool)
    assert np.all(np64(gpu["hidden"])[~us] == 0.0)
    if "position_update" in gpu:
        assert np.all(np64(gpu["position_update"])[~us] == 0.0)
    if "token_output" in gpu:
        T = w.dims["T"]
        a2t = w.structure["atom_to_token"].numpy()
        cnt = np.zeros((w.dims["B"], T), np.int64)
        for b in range(w.dims["B"]):
            t = a2t[b][us[b]]
            np.add.at(cnt[b], t, 1)
        to = np64(gpu["token_output"])
        assert np.all(to[cnt == 0] == 0.0)
        return cnt
    return None


def compare_block(w, gpu, ref, rows=None, tokens=None):
    """Compare every output; `rows` ([B,A] bool) / `tokens` ([B,T] bool)
    restrict to the rows the oracle computed."""
    rtol = RTOL[w.dtype]
    hid_w = rows if rows is not None else None
    assert_close("hidden", np64(gpu["hidden"]), ref["hidden"], rtol, hid_w)
    att = np64(gpu["attention"])
    if rows is not None:
        m = np.broadcast_to(rows[:, None, :, None], att.shape)
        assert_close_rel("attention", att, ref["attention"], rtol, m)
    else:
        assert_close_rel("attention", att, ref["attention"], rtol)
    if "token_output" in gpu:
        assert_close("token_output", np64(gpu["token_output"]), ref["token_output"],
                     rtol, tokens)
    else:
        assert_close("position_update", np64(gpu["position_update"]),
                     ref["position_update"], rtol, hid_w)
