"""GPU parity of the backward pass: atom_attn_backward and
atom_attn_slot_attention_backward (through the C ABI) against the fp64
gradient oracle (oracle/block_grad.py, itself pinned to finite differences
of the C oracle) on the same seeded inputs.

Tolerance: the backward pass computes in fp32 whatever the input storage
(bf16 inputs are widened exactly), so every gradient tensor is held to
|gpu - oracle| <= 1e-4 * (|oracle| + rms(oracle)) -- the fp32 bar of the
forward parity tests: fp32 sums of up to ~10^5 terms (parameter gradients
over every atom) carry relative errors near 1e-6, and the normalisation
and softmax backward steps cancel at most a few digits more. Exact zeros
the method fixes (unusable atoms, slots that are not allowed) are compared
bit-exactly.

The encoder pooling applies ReLU to each atom's pooled projection, whose
derivative is undefined at 0. A projection within fp32 rounding of 0 can
land on either side in the GPU's fp32 arithmetic and the oracle's fp64, and
the two are then both valid but different gradients (the whole backward of
that atom and its window changes). The upstream token gradient is therefore
zeroed on each (token, channel) with an atom whose oracle projection lies
within 1e-4 rms of the kink: no gradient depends on the side taken there.
"""
import numpy as np
import pytest
import torch

from _parity import assert_close, np64
from oracle import block_grad
from windowed_atom_attention_amd import block_backward, slot_attention_backward
from windowed_atom_attention_amd.workloads import make_workload

pytestmark = pytest.mark.gpu

RTOL = 1e-4


def _upstream(w, seed=21, which=("hidden", "attention", "pooled")):
    g = torch.Generator().manual_seed(seed)
    d = w.dims
    B, A, T, C, H, K, U = (d[k] for k in "B A T C H K U".split())
    up = {}
    if "hidden" in which:
        up["hidden"] = torch.randn((B, A, C), generator=g)
    if "attention" in which:
        up["attention"] = torch.randn((B, H, A, K), generator=g)
    if "pooled" in which:
        if w.stage == "encoder":
            up["token_output"] = torch.randn((B, T, U), generator=g)
        else:
            up["position_update"] = torch.randn((B, A, 3), generator=g)
    return up


def _kink_safe(w, up):
    """Zero d_token_output[b, t, u] where a usable atom of token t has its
    oracle projection (hidden @ w_pool, fp64) within 1e-4 rms of the ReLU
    kink."""
    if w.stage != "encoder" or "token_output" not in up:
        return up
    f64 = lambda d: {k: v.to(torch.float64) for k, v in d.items()}
    out = block_grad.block_forward(f64(w.activations), f64(w.parameters), w.masks, w.structure,
                                   eps=w.eps, style=w.style, stage=w.stage, radius=w.radius)
    proj = out["hidden"].detach() @ w.parameters["w_pool"].to(torch.float64)
    a2t = w.structure["atom_to_token"]
    T = w.dims["T"]
    inr = (a2t >= 0) & (a2t < T)
    usable = w.masks["valid"] & inr & torch.gather(w.masks["token_valid"], 1, a2t.clamp(0, T - 1))
    rms = proj[usable].pow(2).mean().sqrt()
    near = (proj.abs() <= 1e-4 * rms) & usable[..., None]
    b, n, u = torch.nonzero(near, as_tuple=True)
    t = a2t[b, n]
    up = dict(up)
    up["token_output"] = up["token_output"].clone()
    up["token_output"][b, t, u] = 0.0
    return up


def _gpu_backward(w, up, **kw):
    g = w.to("cuda")
    din, dpar = block_backward(g.activations, g.parameters, g.masks, g.structure,
                               {k: v.cuda() for k, v in up.items()}, eps=w.eps, style=w.style,
                               stage=w.stage, radius=w.radius, **kw)
    torch.cuda.synchronize()
    return din, dpar


def _compare(w, din, dpar, ref_in, ref_par):
    assert set(din) == set(ref_in), (sorted(din), sorted(ref_in))
    assert set(dpar) == set(ref_par), (sorted(dpar), sorted(ref_par))
    for k in sorted(ref_in):
        assert_close("d_" + k, np64(din[k]), ref_in[k].numpy(), RTOL)
    for k in sorted(ref_par):
        assert_close("d_" + k, np64(dpar[k]), ref_par[k].numpy(), RTOL)
    # exact zeros: unusable atoms' inputs; pair rows of slots not allowed
    valid = w.masks["valid"].numpy()
    assert np.all(np64(din["atom"])[~valid] == 0.0)
    assert np.all(np64(din["condition"])[~valid] == 0.0)
    if "pair" in din:
        assert np.all(np64(din["pair"])[~valid] == 0.0)
        miss = (w.structure["key_index"] < 0) | (w.structure["key_index"] >= w.dims["A"])
        assert np.all(np64(din["pair"])[miss.numpy()] == 0.0)


CASES = [
    ("0", {}),
    ("0", dict(stage="decoder")),
    ("0", dict(style="esmfold2")),
    ("0", dict(style="esmfold2", stage="decoder", dtype=torch.bfloat16)),
    ("1", dict(A=300)),
    ("2", dict(A=300)),
    ("3", dict(B=2, A=400)),
    ("4a", dict(A=500)),
    ("4b", dict(A=500)),
    ("1", dict(A=200, dtype=torch.bfloat16, stage="decoder")),
    ("0", dict(A=300, K=200, dtype=torch.bfloat16, stage="decoder")),
    ("0", dict(A=150, H=4, D=64, V=16, K=40)),
    ("0", dict(A=200, K=48, style="esmfold2", H=8, D=16)),
    ("0", dict(A=120, H=2, D=8, K=24, style="esmfold2", stage="decoder")),
    ("0", dict(A=100, C=48, S=40, M=72, U=20)),
    # 768 query blocks of 16: the block form of the slot step's query side
    ("4a", dict(A=12288)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=["%s-%s" % (n, "-".join(
    "%s=%s" % (k, str(v).replace("torch.", "")) for k, v in kw.items())) for n, kw in CASES])
def test_block_backward_matches_oracle(name, kw):
    w = make_workload(name, rope="distinct", **kw)
    print("case", name, kw, w.style, w.stage, w.dtype, flush=True)
    up = _kink_safe(w, _upstream(w))
    _, ref_in, ref_par = block_grad.block_backward(w.activations, w.parameters, w.masks,
                                                   w.structure, up, eps=w.eps, style=w.style,
                                                   stage=w.stage, radius=w.radius)
    din, dpar = _gpu_backward(w, up)
    _compare(w, din, dpar, ref_in, ref_par)


def test_block_backward_partial_upstream_and_subsets():
    """Missing upstream gradients are zeros; requesting a subset of the
    gradients gives the same values for those."""
    w = make_workload("0", stage="decoder")
    up = _upstream(w, which=("hidden",))
    _, ref_in, ref_par = block_grad.block_backward(w.activations, w.parameters, w.masks,
                                                   w.structure, up, eps=w.eps, style=w.style,
                                                   stage=w.stage, radius=w.radius)
    din, dpar = _gpu_backward(w, up)
    _compare(w, din, dpar, ref_in, ref_par)
    din2, dpar2 = _gpu_backward(w, up, inputs=("atom",), params=("w_q", "w_readout"))
    assert set(din2) == {"atom"} and set(dpar2) == {"w_q", "w_readout"}
    assert torch.equal(din2["atom"], din["atom"])
    assert torch.equal(dpar2["w_q"], dpar["w_q"])
    assert torch.equal(dpar2["w_readout"], dpar["w_readout"])
    assert float(dpar2["w_readout"].abs().max()) == 0.0  # no position_update gradient


def test_block_backward_is_deterministic():
    w = make_workload("4a", A=700)
    up = _kink_safe(w, _upstream(w))
    a_in, a_par = _gpu_backward(w, up)
    b_in, b_par = _gpu_backward(w, up)
    for k in a_in:
        assert torch.equal(a_in[k], b_in[k]), k
    for k in a_par:
        assert torch.equal(a_par[k], b_par[k]), k


def test_block_backward_full_size_headline_workload():
    """The AF3 encoder fp32 workload at its full size (A=4608, K=128), every
    gradient against the oracle."""
    w = make_workload("1")
    up = _kink_safe(w, _upstream(w))
    _, ref_in, ref_par = block_grad.block_backward(w.activations, w.parameters, w.masks,
                                                   w.structure, up, eps=w.eps, style=w.style,
                                                   stage=w.stage, radius=w.radius)
    din, dpar = _gpu_backward(w, up)
    _compare(w, din, dpar, ref_in, ref_par)


def _slot_inputs(style, B=2, A=70, K=24, H=2, D=16, V=8, seed=4, hub=None, dtype=torch.float32,
                 local=None):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, A, H * D), generator=g)
    k = torch.randn((B, A, H * D), generator=g)
    v = torch.randn((B, A, H * D), generator=g)
    usable = torch.rand((B, A), generator=g) < 0.9
    ki = torch.randint(-2, A + 2, (B, A, K), generator=g)
    if local is not None:
        # key ids within +-local of the query (a narrow band per 16-query
        # block), except in every eighth block of queries, which keeps the
        # scattered ids (a wide band)
        a = torch.arange(A).view(1, A, 1)
        near = (a + torch.randint(-local, local + 1, (B, A, K), generator=g)).clamp(-1, A)
        far_block = ((torch.arange(A) // 16) % 8 == 3).view(1, A, 1)
        ki = torch.where(far_block, ki, near)
    ki[:, :, 1] = ki[:, :, 0]                     # repeats within a row
    if hub is not None:
        ki[:, :, 2:2 + hub] = 5                   # one key selected by many slots
    wm = torch.rand((B, A, K), generator=g) < 0.9
    d_att = torch.randn((B, H, A, K), generator=g)
    d_o = torch.randn((B, A, H * D), generator=g)
    extra = {}
    if style == "af3":
        extra = dict(pair=torch.randn((B, A, K, V), generator=g).to(dtype),
                     pair_scale=(1 + 0.1 * torch.randn((V,), generator=g)).to(dtype),
                     w_pair=(0.5 * torch.randn((V, H), generator=g)).to(dtype))
        junk = ~usable[..., None, None].expand(B, A, K, V)
        extra["pair"] = torch.where(junk, torch.full_like(extra["pair"], float("nan")),
                                    extra["pair"])
    return q, k, v, usable, ki, wm, d_att, d_o, extra, H


SLOT_CASES = [
    ("af3", {}), ("esmfold2", {}),
    ("af3", dict(dtype=torch.bfloat16, K=40, V=16, H=4, D=32)),
    ("esmfold2", dict(K=300, H=4, D=8, A=50)),
    ("af3", dict(D=64, H=4, K=17)),
    # a key selected by thousands of slots (lists beyond the in-register
    # and the LDS sort paths)
    ("esmfold2", dict(hub=20, A=120, K=30)),
    ("af3", dict(hub=3, A=200, K=16)),
    # 768+ query blocks: the block form, with some blocks queued for the
    # per-query kernel (scattered ids) and repeated keys
    ("af3", dict(B=48, A=256, K=64, H=4, D=32, V=16, local=40)),
    ("esmfold2", dict(B=48, A=260, K=48, H=4, D=16, local=30)),
    ("af3", dict(B=24, A=520, K=128, H=2, D=64, V=8, local=56, dtype=torch.bfloat16)),
]


@pytest.mark.parametrize("style,kw", SLOT_CASES)
def test_slot_backward_matches_oracle(style, kw):
    q, k, v, usable, ki, wm, d_att, d_o, extra, H = _slot_inputs(style, **kw)
    radius = 30 if style == "esmfold2" else -1
    print("slot case", style, kw, flush=True)
    ref = block_grad.slot_backward(q, k, v, usable, ki, wm, d_att, d_o, style=style,
                                   radius=radius, heads=H, **extra)
    cu = lambda x: x.cuda() if isinstance(x, torch.Tensor) else x
    got = slot_attention_backward(cu(q), cu(k), cu(v), cu(usable), cu(ki), cu(wm), cu(d_o), H,
                                  d_attention=cu(d_att), style=style, radius=radius,
                                  **{n: cu(t) for n, t in extra.items()})
    names = ["attention", "o", "dq", "dk", "dv"]
    if style == "af3":
        names += ["d_pair", "d_pair_scale", "d_w_pair"]
    for n in names:
        assert_close(n, np64(got[n]), ref[n].numpy(), RTOL)
    # exact zeros: rows of unusable atoms
    bad = ~usable.numpy()
    for n in ("dq", "dk", "dv", "o"):
        assert np.all(np64(got[n])[bad] == 0.0), n
    if style == "af3":
        assert np.all(np64(got["d_pair"])[bad] == 0.0)


def test_slot_backward_without_attention_gradient_and_repeat_bits():
    q, k, v, usable, ki, wm, d_att, d_o, extra, H = _slot_inputs("af3", hub=2)
    ref = block_grad.slot_backward(q, k, v, usable, ki, wm, None, d_o, style="af3", heads=H,
                                   **extra)
    cu = lambda x: x.cuda()
    args = (cu(q), cu(k), cu(v), cu(usable), cu(ki), cu(wm), cu(d_o), H)
    ex = {n: cu(t) for n, t in extra.items()}
    a = slot_attention_backward(*args, style="af3", **ex)
    b = slot_attention_backward(*args, style="af3", **ex)
    for n in ("dq", "dk", "dv", "d_pair", "d_pair_scale", "d_w_pair"):
        assert_close(n, np64(a[n]), ref[n].numpy(), RTOL)
        assert torch.equal(a[n], b[n]), n


def test_block_form_is_deterministic():
    """The block forms of the slot step (768+ query blocks) add each query's
    weights and logit gradients into their LDS tiles in a fixed order:
    repeated calls give identical bits, also with queued wide blocks."""
    q, k, v, usable, ki, wm, d_att, d_o, extra, H = _slot_inputs(
        "af3", B=48, A=256, K=64, H=4, D=32, V=16, local=40)
    cu = lambda x: x.cuda()
    args = (cu(q), cu(k), cu(v), cu(usable), cu(ki), cu(wm), cu(d_o), H)
    ex = {n: cu(t) for n, t in extra.items()}
    a = slot_attention_backward(*args, d_attention=cu(d_att), style="af3", **ex)
    b = slot_attention_backward(*args, d_attention=cu(d_att), style="af3", **ex)
    for n in a:
        assert torch.equal(a[n], b[n]), n
    w = make_workload("4a", A=12288)
    up = _upstream(w)
    a_in, a_par = _gpu_backward(w, up)
    b_in, b_par = _gpu_backward(w, up)
    for kk in a_in:
        assert torch.equal(a_in[kk], b_in[kk]), kk
    for kk in a_par:
        assert torch.equal(a_par[kk], b_par[kk]), kk
