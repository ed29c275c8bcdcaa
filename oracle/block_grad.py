"""fp64 CPU gradients of the windowed atom-attention block (encoder and
decoder stage, AF3 and ESMFold2 style).

TEST INFRASTRUCTURE ONLY. Only the test suite imports this module; the
product library never does, and this module imports nothing from the
product. It shares no code with the HIP kernels.

Sources (all "Required behavior" unless stated):
  [W]  windowed_atom_attention -- Local atom attention, encoder pooling and
       decoder skip/readout (also the repeated-selection rule: a key atom
       chosen by several query slots receives the sum of their gradients)
  [AF] AlphaFold 3 Atom Attention Encoder (its Starter code grades values,
       shapes and gradients)
  [EF] ESMFold 2 Atom Attention Encoder

What a gradient is needs no reading of the pages: it is the derivative of
the block's outputs. So this file writes the block's forward once more as
plain fp64 torch array steps, in the pages' order, and lets torch's
reverse-mode differentiation (a library primitive, like a matmul) take the
derivative of a scalar loss <outputs, upstream gradients>. The forward here
is pinned to the C oracle (oracle.c) value by value, and every gradient is
pinned to central finite differences of the C oracle's forward, in the
test suite.

Selections are written so that no discarded value (NaN/Inf payloads of
unusable atoms, pair rows of slots that are not allowed, rows of invalid
tokens) enters any arithmetic, forward or backward: they are replaced by
zeros before use, so their gradients are exactly zero.
"""
from __future__ import annotations

import math

import torch

__all__ = ["block_forward", "block_backward", "slot_backward", "FLOAT_INPUTS"]

F64 = torch.float64

# float inputs of the block that receive gradients, per style/stage
FLOAT_INPUTS = {
    ("af3", "encoder"): ["atom", "condition", "pair"],
    ("af3", "decoder"): ["atom", "condition", "pair", "token"],
    ("esmfold2", "encoder"): ["atom", "condition", "rope_cos", "rope_sin"],
    ("esmfold2", "decoder"): ["atom", "condition", "rope_cos", "rope_sin", "token"],
}


def _ln(x, eps):
    """Population LayerNorm over the last axis, no affine, eps in the root
    ([W] AF3 style bullet)."""
    mean = x.mean(dim=-1, keepdim=True)
    var = ((x - mean) ** 2).mean(dim=-1, keepdim=True)
    return (x - mean) / torch.sqrt(var + eps)


def _rms(x, eps):
    """x / sqrt(mean(x^2) + eps) over the last axis ([W] ESMFold2 bullets)."""
    return x / torch.sqrt((x * x).mean(dim=-1, keepdim=True) + eps)


def _rotary(x, cos, sin):
    """Half-split rotary with full-width tables: x*cos + [-x2, x1]*sin
    ([W] ESMFold2 rotary bullet)."""
    h = x.shape[-1] // 2
    rot = torch.cat([-x[..., h:], x[..., :h]], dim=-1)
    return x * cos + rot * sin


def _zero(x):
    return torch.zeros((), dtype=x.dtype)


def block_forward(acts, params, masks, structure, eps=1e-5, style="af3",
                  stage="encoder", radius=-1):
    """The block's outputs from fp64 tensors (acts/params may require grad):
    dict with hidden [B,A,C], attention [B,H,A,K] and token_output [B,T,U]
    (encoder) or position_update [B,A,3] (decoder)."""
    p = params
    atom, cond = acts["atom"], acts["condition"]
    B, A, C = atom.shape
    S = cond.shape[-1]
    valid = masks["valid"].bool()
    token_valid = masks["token_valid"].bool()
    wm = masks["window_mask"].bool()
    a2t = structure["atom_to_token"].long()
    ki = structure["key_index"].long()
    T = token_valid.shape[-1]
    K = ki.shape[-1]
    HD = p["w_q"].shape[-1]
    if style == "af3":
        H = p["w_pair"].shape[-1]
    else:
        H = HD // acts["rope_cos"].shape[-1]
    D = HD // H
    bidx = torch.arange(B)[:, None]

    # usability and sanitising ([W]: usable = valid, token in range, token valid)
    in_range = (a2t >= 0) & (a2t < T)
    tcl = a2t.clamp(0, T - 1)
    usable = valid & in_range & torch.gather(token_valid, 1, tcl)
    u = usable[..., None]
    x0 = torch.where(u, atom, _zero(atom))
    if stage == "decoder":
        # decoder entry: skip plus the gathered token projection (bias-free)
        tok = torch.where(token_valid[..., None], acts["token"], _zero(acts["token"]))
        tp = tok @ p["w_token"]                                 # [B, T, C]
        x0 = torch.where(u, x0 + tp[bidx, tcl], _zero(x0))
    c = torch.where(u, cond, _zero(cond))

    # conditioning and the modulated norms
    if style == "af3":
        ch = _ln(c, eps)
        sig, mu = [], []
        for j in range(3):
            cj = ch * p["cond_scale"][j]
            sig.append(torch.sigmoid(cj @ p["w_scale"][j] + p["b_scale"][j]))
            mu.append(cj @ p["w_shift"][j])
        g_att = torch.sigmoid(c @ p["w_residual_gate"][0] + p["b_residual_gate"][0])
        g_tr = torch.sigmoid(c @ p["w_residual_gate"][1] + p["b_residual_gate"][1])
        xn = _ln(x0, eps)
        q_in = xn * sig[0] + mu[0]
        kv_in = xn * sig[1] + mu[1]
    else:
        mods = torch.nn.functional.silu(c) @ p["w_mod"].reshape(S, 6 * C)
        m = [mods[..., i * C:(i + 1) * C] for i in range(6)]
        q_in = _rms(x0, eps) * (1.0 + m[1]) + m[0]
        kv_in = q_in
        g_att, g_tr = m[2], m[5]

    # projections (+ESMFold2 per-head RMS and rotary)
    Q = q_in @ p["w_q"]
    if style == "af3":
        Q = Q + p["b_q"]
    Kp = kv_in @ p["w_k"]
    Vp = kv_in @ p["w_v"]
    G = torch.sigmoid(q_in @ p["w_value_gate"])
    Q = Q.reshape(B, A, H, D)
    Kp = Kp.reshape(B, A, H, D)
    Vp = Vp.reshape(B, A, H, D)
    if style == "esmfold2":
        cs = acts["rope_cos"][:, :, None, :]
        sn = acts["rope_sin"][:, :, None, :]
        Q = _rotary(_rms(Q, eps), cs, sn)
        Kp = _rotary(_rms(Kp, eps), cs, sn)

    # slot permission ([W]): id in range, both atoms usable, window_mask, radius
    inr = (ki >= 0) & (ki < A)
    jc = ki.clamp(0, A - 1)
    usable_k = torch.gather(usable, 1, jc.reshape(B, A * K)).reshape(B, A, K)
    allowed = usable[..., None] & inr & usable_k & wm
    if radius >= 0:
        allowed = allowed & ((jc - torch.arange(A)[None, :, None]).abs() <= radius)

    Kg = Kp[bidx[..., None], jc]                                # [B, A, K, H, D]
    Vg = Vp[bidx[..., None], jc]
    logits = torch.einsum("bahd,bakhd->bahk", Q, Kg) / math.sqrt(D)
    if style == "af3":
        pr = torch.where(allowed[..., None], acts["pair"], _zero(acts["pair"]))
        beta = (_ln(pr, eps) * p["pair_scale"]) @ p["w_pair"]   # [B, A, K, H]
        logits = logits + beta.permute(0, 1, 3, 2)
    mask = allowed[:, :, None, :]                               # [B, A, 1, K]
    # masked softmax over the allowed slots; a row with none is all zeros
    lm = torch.where(mask, logits, torch.full((), -math.inf, dtype=F64))
    mx = lm.max(dim=-1, keepdim=True).values
    mx = torch.where(torch.isfinite(mx), mx, torch.zeros((), dtype=F64)).detach()
    e = torch.where(mask, torch.exp(torch.where(mask, logits, _zero(logits)) - mx),
                    _zero(logits))
    den = e.sum(dim=-1, keepdim=True)
    P = e / torch.where(den > 0, den, torch.ones((), dtype=F64))
    o = torch.einsum("bahk,bakhd->bahd", P, Vg).reshape(B, A, HD)
    attention = P.permute(0, 2, 1, 3)                           # [B, H, A, K]

    # value gate, output projection, gated residual
    x1 = x0 + g_att * ((o * G) @ p["w_attention_out"])
    # transition on the new state, gated residual, mask
    if style == "af3":
        z = _ln(x1, eps) * sig[2] + mu[2]
    else:
        z = _rms(x1, eps) * (1.0 + m[4]) + m[3]
    hh = torch.nn.functional.silu(z @ p["w_ff_gate"]) * (z @ p["w_ff_up"])
    hidden = torch.where(u, x1 + g_tr * (hh @ p["w_ff_out"]), _zero(x1))

    out = {"hidden": hidden, "attention": attention}
    if stage == "encoder":
        # per-token mean of ReLU(hidden @ w_pool) over usable assigned atoms
        proj = torch.relu(hidden @ p["w_pool"])
        U = proj.shape[-1]
        bb = bidx.expand(B, A)[usable]
        tt = tcl[usable]
        sums = torch.zeros((B, T, U), dtype=F64).index_put((bb, tt), proj[usable],
                                                           accumulate=True)
        cnt = torch.zeros((B, T), dtype=F64).index_put(
            (bb, tt), torch.ones(len(tt), dtype=F64), accumulate=True)
        out["token_output"] = sums / torch.where(cnt > 0, cnt, torch.ones((), dtype=F64))[..., None]
    else:
        lnh = _ln(hidden, eps) * p["readout_scale"]
        if style == "esmfold2":
            lnh = lnh + p["readout_bias"]
        out["position_update"] = torch.where(u, lnh @ p["w_readout"], _zero(hidden[..., :3]))
    return out


def _f64(x):
    return x.detach().to("cpu").to(F64).clone()


def block_backward(acts, params, masks, structure, grads_out, eps=1e-5, style="af3",
                   stage="encoder", radius=-1):
    """Gradients of every float input and parameter of the block.

    grads_out: upstream gradients of the outputs, by output name (hidden,
    attention, token_output / position_update; a missing one is zero).
    Returns (outputs, input_grads, param_grads), all fp64 CPU tensors: the
    derivative of sum over outputs of <output, upstream gradient>."""
    a = {k: _f64(v).requires_grad_(k in FLOAT_INPUTS[(style, stage)])
         for k, v in acts.items()}
    pr = {k: _f64(v).requires_grad_(True) for k, v in params.items() if v is not None}
    ms = {k: v.detach().to("cpu") for k, v in masks.items()}
    st = {k: v.detach().to("cpu") for k, v in structure.items()}
    out = block_forward(a, pr, ms, st, eps=eps, style=style, stage=stage, radius=radius)
    loss = torch.zeros((), dtype=F64)
    for name, g in grads_out.items():
        if g is not None and name in out:
            loss = loss + (out[name] * _f64(g)).sum()
    leaves = [(("in", k), v) for k, v in a.items() if v.requires_grad]
    leaves += [(("par", k), v) for k, v in pr.items()]
    gs = torch.autograd.grad(loss, [v for _, v in leaves], allow_unused=True)
    din, dpar = {}, {}
    for ((kind, k), v), g in zip(leaves, gs):
        g = torch.zeros_like(v) if g is None else g
        (din if kind == "in" else dpar)[k] = g.detach()
    return {k: v.detach() for k, v in out.items()}, din, dpar


def slot_backward(q, k, v, usable, key_index, window_mask, d_attention, d_o, eps=1e-5,
                  style="af3", radius=-1, pair=None, pair_scale=None, w_pair=None, heads=1):
    """Gradients of the slot-attention step alone ([W]: masked softmax over
    the allowed slots of Q.K/sqrt(D) (+ AF3 pair bias), o = sum_k w_k V[key_k]).

    q, k, v [B,A,H*D]; d_attention [B,H,A,K] (or None), d_o [B,A,H*D].
    Returns dict dq, dk, dv (and d_pair, d_pair_scale, d_w_pair for AF3)."""
    qq, kk, vv = (_f64(x).requires_grad_(True) for x in (q, k, v))
    B, A, HD = qq.shape
    H = int(heads)
    D = HD // H
    us = usable.detach().to("cpu").bool()
    ki = key_index.detach().to("cpu").long()
    wm = window_mask.detach().to("cpu").bool()
    K = ki.shape[-1]
    bidx = torch.arange(B)[:, None, None]
    inr = (ki >= 0) & (ki < A)
    jc = ki.clamp(0, A - 1)
    usable_k = torch.gather(us, 1, jc.reshape(B, A * K)).reshape(B, A, K)
    allowed = us[..., None] & inr & usable_k & wm
    if radius >= 0:
        allowed = allowed & ((jc - torch.arange(A)[None, :, None]).abs() <= radius)
    Q = qq.reshape(B, A, H, D)
    Kg = kk.reshape(B, A, H, D)[bidx, jc]
    Vg = vv.reshape(B, A, H, D)[bidx, jc]
    logits = torch.einsum("bahd,bakhd->bahk", Q, Kg) / math.sqrt(D)
    extra = []
    if style == "af3":
        pp = _f64(pair).requires_grad_(True)
        ps = _f64(pair_scale).requires_grad_(True)
        wp = _f64(w_pair).requires_grad_(True)
        extra = [pp, ps, wp]
        prs = torch.where(allowed[..., None], pp, torch.zeros((), dtype=F64))
        beta = (_ln(prs, eps) * ps) @ wp
        logits = logits + beta.permute(0, 1, 3, 2)
    mask = allowed[:, :, None, :]
    lm = torch.where(mask, logits, torch.full((), -math.inf, dtype=F64))
    mx = lm.max(dim=-1, keepdim=True).values
    mx = torch.where(torch.isfinite(mx), mx, torch.zeros((), dtype=F64)).detach()
    e = torch.where(mask, torch.exp(torch.where(mask, logits, torch.zeros((), dtype=F64)) - mx),
                    torch.zeros((), dtype=F64))
    den = e.sum(dim=-1, keepdim=True)
    P = e / torch.where(den > 0, den, torch.ones((), dtype=F64))
    o = torch.einsum("bahk,bakhd->bahd", P, Vg).reshape(B, A, HD)
    att = P.permute(0, 2, 1, 3)
    loss = (o * _f64(d_o)).sum()
    if d_attention is not None:
        loss = loss + (att * _f64(d_attention)).sum()
    gs = torch.autograd.grad(loss, [qq, kk, vv] + extra, allow_unused=True)
    gs = [torch.zeros_like(x) if g is None else g for x, g in zip([qq, kk, vv] + extra, gs)]
    res = {"dq": gs[0], "dk": gs[1], "dv": gs[2], "attention": att.detach(), "o": o.detach()}
    if style == "af3":
        res.update(d_pair=gs[3], d_pair_scale=gs[4], d_w_pair=gs[5])
    return res
