"""Pins of the fp64 pair-operator oracle (oracle/pair_ops.py) against things
other than itself: the worked examples of "ESMFold Single-to-Pair Features"
and "Tied Pair Row Attention" (tests/golden/, cited there), special cases
with closed forms, reductions to torch's scaled_dot_product_attention and
layer_norm, invariants, and brute-force scalar loops on tiny inputs written
in the untransposed coordinates."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import pair_ops as P

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F64 = torch.float64


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------- single-to-pair

def test_single_to_pair_worked_example():
    g = _load("esmfold_single_to_pair_worked_example.json")
    p = g["parameters"]
    pf, out = P.single_to_pair(g["x"], np.array(g["mask"]), p["weight"], p["bias"],
                               p["norm_scale"], p["norm_bias"], p["out_weight"],
                               p["out_bias"], eps=g["eps"], output_norm=g["output_norm"])
    np.testing.assert_allclose(pf, g["expected_pair_features"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, g["expected_output"], rtol=0, atol=1e-12)


def _s2p_inputs(seed, B=2, N=7, C=6, H=3, D=5, absent=(1, 4)):
    r = _rng(seed)
    x = r.normal(size=(B, N, C)) * 1.5 + 0.3
    mask = np.ones((B, N), bool)
    for i in absent:
        mask[:, i] = False
    x[~mask] = np.nan  # absent payloads are junk
    par = dict(weight=r.normal(size=(C, 2 * H)), bias=r.normal(size=2 * H),
               norm_scale=1 + 0.2 * r.normal(size=C), norm_bias=0.3 * r.normal(size=C),
               out_weight=r.normal(size=(2 * H, D)), out_bias=r.normal(size=D),
               output_scale=1 + 0.2 * r.normal(size=D), output_bias=0.3 * r.normal(size=D))
    return x, mask, par


def _s2p(x, mask, par, eps=1e-5, output_norm=False, rows=None):
    return P.single_to_pair(x, mask, par["weight"], par["bias"], par["norm_scale"],
                            par["norm_bias"], par["out_weight"], par["out_bias"], eps=eps,
                            output_norm=output_norm, output_scale=par["output_scale"],
                            output_bias=par["output_bias"], rows=rows)


def test_single_to_pair_bruteforce_loops():
    """Scalar loops over (b, i, j, channel) with torch's layer_norm for the
    token normalisation; absent endpoints give exact zeros."""
    x, mask, par = _s2p_inputs(1, B=1, N=5, C=4, H=2, D=3, absent=(2,))
    eps = 0.7
    for on in (False, True):
        pf, out = _s2p(x, mask, par, eps=eps, output_norm=on)
        xt = torch.from_numpy(np.where(mask[..., None], x, 0.0))
        xn = F.layer_norm(xt, (4,), torch.from_numpy(par["norm_scale"]),
                          torch.from_numpy(par["norm_bias"]), eps=eps).numpy()
        N, H, D = 5, 2, 3
        for i, j in itertools.product(range(N), range(N)):
            if not (mask[0, i] and mask[0, j]):
                assert np.all(pf[0, i, j] == 0.0) and np.all(out[0, i, j] == 0.0)
                continue
            y_i = [sum(xn[0, i, c] * par["weight"][c, o] for c in range(4)) + par["bias"][o]
                   for o in range(2 * H)]
            y_j = [sum(xn[0, j, c] * par["weight"][c, o] for c in range(4)) + par["bias"][o]
                   for o in range(2 * H)]
            k_i, q_j = y_i[H:], y_j[:H]
            feat = [k_i[h] * q_j[h] for h in range(H)] + [q_j[h] - k_i[h] for h in range(H)]
            np.testing.assert_allclose(pf[0, i, j], feat, rtol=0, atol=1e-12)
            o = [sum(feat[c] * par["out_weight"][c, d] for c in range(2 * H)) + par["out_bias"][d]
                 for d in range(D)]
            if on:
                m = sum(o) / D
                v = sum((t - m) ** 2 for t in o) / D
                o = [(t - m) / math.sqrt(v + eps) * par["output_scale"][d] + par["output_bias"][d]
                     for d, t in enumerate(o)]
            np.testing.assert_allclose(out[0, i, j], o, rtol=0, atol=1e-12)


def test_single_to_pair_zero_norm_scale_closed_form():
    """norm_scale = 0: every present token normalises to norm_bias, so q and
    k are the same for every token and every present pair carries
    [k * q, q - k] with y = norm_bias @ weight + bias."""
    x, mask, par = _s2p_inputs(2)
    par["norm_scale"] = np.zeros_like(par["norm_scale"])
    pf, out = _s2p(x, mask, par)
    y = par["norm_bias"] @ par["weight"] + par["bias"]
    H = y.size // 2
    q, k = y[:H], y[H:]
    exp = np.concatenate([k * q, q - k])
    both = mask[:, :, None] & mask[:, None, :]
    np.testing.assert_allclose(pf[both], np.broadcast_to(exp, pf[both].shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[both], np.broadcast_to(exp @ par["out_weight"] + par["out_bias"],
                                                          out[both].shape), rtol=0, atol=1e-12)


def test_single_to_pair_direction_and_head():
    """With the q and k halves of the projection equal (q = k), the product
    channels are symmetric in (i, j) and the difference channels
    antisymmetric; the output is the pair features @ out_weight + out_bias;
    with output_norm the output is torch's layer_norm of that."""
    x, mask, par = _s2p_inputs(3)
    H = par["weight"].shape[1] // 2
    par["weight"][:, H:] = par["weight"][:, :H]
    par["bias"][H:] = par["bias"][:H]
    pf, out = _s2p(x, mask, par)
    np.testing.assert_allclose(pf[..., :H], np.swapaxes(pf[..., :H], 1, 2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(pf[..., H:], -np.swapaxes(pf[..., H:], 1, 2), rtol=0, atol=1e-12)
    both = mask[:, :, None] & mask[:, None, :]
    lin = pf @ par["out_weight"] + par["out_bias"]
    np.testing.assert_allclose(out[both], lin[both], rtol=0, atol=1e-12)
    _, outn = _s2p(x, mask, par, output_norm=True)
    ref = F.layer_norm(torch.from_numpy(lin), (lin.shape[-1],),
                       torch.from_numpy(par["output_scale"]),
                       torch.from_numpy(par["output_bias"]), eps=1e-5).numpy()
    np.testing.assert_allclose(outn[both], ref[both], rtol=0, atol=1e-12)
    assert np.all(outn[~both] == 0.0)


def test_single_to_pair_rows_and_junk():
    """A row selection returns those rows of the full result; NaN payloads
    of absent tokens never reach an output."""
    x, mask, par = _s2p_inputs(4)
    pf, out = _s2p(x, mask, par, output_norm=True)
    assert np.all(np.isfinite(pf)) and np.all(np.isfinite(out))
    rows = np.array([0, 3, 6])
    pr, orow = _s2p(x, mask, par, output_norm=True, rows=rows)
    np.testing.assert_array_equal(pr, pf[:, rows])
    np.testing.assert_array_equal(orow, out[:, rows])


# ------------------------------------------------- tied pair row attention

def _tied(feat, bfeat, par, eps):
    return P.tied_row_attention(feat, bfeat, par["norm_scale"], par["norm_bias"],
                                par["bias_norm_scale"], par["bias_norm_bias"], par["w_q"],
                                par["w_k"], par["w_v"], par["w_bias"], par["w_gate"],
                                par["w_out"], par["b_out"], eps=eps)


def test_tied_row_attention_worked_example():
    g = _load("tied_pair_row_attention_worked_example.json")
    ns = {"exp": math.exp, "sqrt": math.sqrt}
    for k, v in g["define"].items():
        ns[k] = eval(v, {"__builtins__": {}}, ns)
    exp = np.array([[[[eval(e, {"__builtins__": {}}, ns) for e in c] for c in row]
                     for row in g["expected"][0]]])
    out = _tied(np.array(g["features"]), np.array(g["bias_features"]),
                {k: np.array(v) for k, v in g["parameters"].items()}, g["eps"])
    np.testing.assert_allclose(out, exp, rtol=0, atol=1e-12)
    val, tol = g["printed"]["p"]
    assert abs(ns["p"] - val) <= tol
    for key, (a, b) in (("out10", (1, 0)), ("out11", (1, 1))):
        val, tol = g["printed"][key]
        assert np.all(np.abs(out[0, a, b] - np.array(val)) <= tol)


def _tied_inputs(seed, B=1, L=5, C=6, Cb=3, H=2, D=3):
    r = _rng(seed)
    feat = r.normal(size=(B, L, L, C))
    bfeat = r.normal(size=(B, L, L, Cb))
    HD = H * D
    par = dict(norm_scale=1 + 0.3 * r.normal(size=C), norm_bias=0.3 * r.normal(size=C),
               bias_norm_scale=1 + 0.3 * r.normal(size=Cb),
               bias_norm_bias=0.3 * r.normal(size=Cb),
               w_q=r.normal(size=(C, HD)), w_k=r.normal(size=(C, HD)),
               w_v=r.normal(size=(C, HD)), w_bias=r.normal(size=(Cb, H)),
               w_gate=r.normal(size=(C, HD)), w_out=r.normal(size=(HD, C)),
               b_out=r.normal(size=C))
    return feat, bfeat, par


def test_tied_row_attention_bruteforce_untransposed():
    """Scalar loops written directly in the original layout, where the
    exchange of axes becomes index bookkeeping: for output position (a, b),
    query b attends over keys j with logits sum_s q(F[b,s]) . k(F[j,s]) /
    sqrt(L*D) + beta(Fb[j,b]), mixes v(F[j,a]), is gated by g(F[a,b]) and
    projected. Catches a transposition slip anywhere in the oracle."""
    L, C, Cb, H, D = 3, 4, 2, 2, 2
    feat, bfeat, par = _tied_inputs(5, L=L, C=C, Cb=Cb, H=H, D=D)
    eps = 0.4
    out = _tied(feat, bfeat, par, eps)
    fn = F.layer_norm(torch.from_numpy(feat[0]), (C,), torch.from_numpy(par["norm_scale"]),
                      torch.from_numpy(par["norm_bias"]), eps=eps).numpy()
    bn = F.layer_norm(torch.from_numpy(bfeat[0]), (Cb,), torch.from_numpy(par["bias_norm_scale"]),
                      torch.from_numpy(par["bias_norm_bias"]), eps=eps).numpy()

    def proj(x, w, h):
        return [sum(x[c] * w[c, h * D + d] for c in range(C)) for d in range(D)]

    for a, b in itertools.product(range(L), range(L)):
        upd = []
        for h in range(H):
            lg = []
            for j in range(L):
                s_ = sum(sum(qq * kk for qq, kk in zip(proj(fn[b, s], par["w_q"], h),
                                                       proj(fn[j, s], par["w_k"], h)))
                         for s in range(L)) / math.sqrt(L * D)
                s_ += sum(bn[j, b, c] * par["w_bias"][c, h] for c in range(Cb))
                lg.append(s_)
            m = max(lg)
            ex = [math.exp(t - m) for t in lg]
            A = [t / sum(ex) for t in ex]
            gate = [1 / (1 + math.exp(-t)) for t in proj(fn[a, b], par["w_gate"], h)]
            for d in range(D):
                u = sum(A[j] * proj(fn[j, a], par["w_v"], h)[d] for j in range(L))
                upd.append(gate[d] * u)
        o = [sum(upd[e] * par["w_out"][e, c] for e in range(H * D)) + par["b_out"][c]
             for c in range(C)]
        np.testing.assert_allclose(out[0, a, b], o, rtol=0, atol=1e-12)


def test_tied_row_attention_reduces_to_sdpa():
    """Features constant along the tied axis (features[i, s] = f_i for every
    s): the tied logits are L * q_i . k_j / sqrt(L*D), i.e. ordinary
    attention with scale sqrt(L/D); every anchor mixes the same values, so
    out[a, b] = (g(f_a) * o_b) @ w_out + b_out with o = torch SDPA."""
    L, C, Cb, H, D = 6, 5, 3, 2, 4
    feat, bfeat, par = _tied_inputs(6, L=L, C=C, Cb=Cb, H=H, D=D)
    f = feat[:, :, :1, :]
    feat = np.broadcast_to(f, feat.shape).copy()
    eps = 1e-5
    out = _tied(feat, bfeat, par, eps)
    fn = F.layer_norm(torch.from_numpy(f[0, :, 0]), (C,), torch.from_numpy(par["norm_scale"]),
                      torch.from_numpy(par["norm_bias"]), eps=eps)          # [L, C]
    bn = F.layer_norm(torch.from_numpy(bfeat[0]), (Cb,),
                      torch.from_numpy(par["bias_norm_scale"]),
                      torch.from_numpy(par["bias_norm_bias"]), eps=eps)     # [L, L, Cb]
    t = lambda k: torch.from_numpy(par[k])
    q = (fn @ t("w_q")).view(L, H, D).transpose(0, 1)
    k = (fn @ t("w_k")).view(L, H, D).transpose(0, 1)
    v = (fn @ t("w_v")).view(L, H, D).transpose(0, 1)
    # bias of query b, key j comes from bias_features[j, b] (axes exchanged)
    beta = (bn.transpose(0, 1) @ t("w_bias")).permute(2, 0, 1)             # [H, b, j]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=beta, scale=math.sqrt(L / D))
    o = o.transpose(0, 1).reshape(L, H * D)                                # [b, HD]
    gate = torch.sigmoid(fn @ t("w_gate"))                                 # [a, HD]
    ref = (gate[:, None, :] * o[None, :, :]) @ t("w_out") + t("b_out")     # [a, b, C]
    np.testing.assert_allclose(out[0], ref.numpy(), rtol=0, atol=1e-12)


def test_tied_row_attention_bias_shift_invariance():
    """Adding a per-(query, head) constant to the pair bias (bias features
    whose projection is constant over the keys) leaves the update unchanged;
    a zero-weight bias equals no bias."""
    feat, bfeat, par = _tied_inputs(7)
    base = _tied(feat, bfeat, dict(par, w_bias=np.zeros_like(par["w_bias"])), 1e-5)
    other = _tied(feat, np.random.default_rng(8).normal(size=bfeat.shape),
                  dict(par, w_bias=np.zeros_like(par["w_bias"])), 1e-5)
    np.testing.assert_allclose(base, other, rtol=0, atol=1e-12)


# ------------------------------------------------------ window table

@pytest.mark.parametrize("A,K,block,radius", [(100, 16, 32, -1), (70, 128, 32, -1),
                                              (200, 128, 32, 48), (97, 24, 8, 5), (5, 4, 2, 0)])
def test_window_table_bruteforce(A, K, block, radius):
    t = P.window_table(2, A, K, block=block, radius=radius)
    assert t.shape == (2, A, K) and t.dtype == np.int64
    for a in range(A):
        b0 = (a // block) * block
        for k in range(K):
            j = b0 - (K - block) // 2 + k
            ok = 0 <= j < A and (radius < 0 or abs(j - a) <= radius)
            assert t[0, a, k] == (j if ok else -1) and t[1, a, k] == t[0, a, k]
    # the window is centred on its block: ids of the block span both sides
    # equally when K - block is even
    if (K - block) % 2 == 0 and radius < 0:
        a = (A // 2 // block) * block
        lo, hi = a - (K - block) // 2, a - (K - block) // 2 + K - 1
        assert (a - lo) == (hi - (a + block - 1))


def test_window_table_matches_workload_tables():
    """Without a radius, the table has the same present ids as the
    windowed tables of the block workloads (which keep out-of-range ids in
    place, missing all the same)."""
    from windowed_atom_attention_amd.workloads import window_table as gen
    g = gen(1, 300, 128).numpy()
    t = P.window_table(1, 300, 128)
    keep = (g >= 0) & (g < 300)
    assert np.array_equal(np.where(keep, g, -1), t)
