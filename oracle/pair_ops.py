"""Plain fp64 CPU oracle of the pair-representation operators and the window
table builder (numpy, straight array steps in the pages' order).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
CPU-baseline leg of ``bench.py`` import this module; the product library
never does, and this module imports nothing from the product. It shares no
code with the HIP kernels.

Sources:
  [S2P]  "ESMFold Single-to-Pair Features" (Required behavior, Worked example)
  [TIED] "Tied Pair Row Attention" (Required behavior, Worked example)
  [WIN]  the windowed slot tables of the atom-attention workloads: each block
         of Q consecutive query atoms sees K consecutive key ids centred on
         the block ("windowed_atom_attention", Required behavior, takes such
         tables as supplied input; this builds one).

Every input is upcast exactly to float64; results are float64.
"""
from __future__ import annotations

import numpy as np

__all__ = ["layer_norm", "single_to_pair", "tied_row_attention", "window_table"]


def _f64(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _bool(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").numpy().astype(bool)
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x).astype(bool)


def layer_norm(x, eps, scale=None, bias=None):
    """Population LayerNorm over the last axis with eps inside the root,
    then the optional affine scale and shift ([S2P], [TIED])."""
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mean) / np.sqrt(var + eps)
    if scale is not None:
        y = y * scale
    if bias is not None:
        y = y + bias
    return y


def sigmoid(z):
    """1/(1+e^-z), written with e^z/(1+e^z) for z < 0 (same value, no
    overflow of e^-z)."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    e = np.exp(z[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def single_to_pair(x, mask, weight, bias, norm_scale, norm_bias, out_weight, out_bias,
                   eps=1e-5, output_norm=False, output_scale=None, output_bias=None,
                   rows=None):
    """[S2P]: returns (pair_features [B,N,N,2H], output [B,N,N,D]).

    x [B,N,C] (tokens), mask [B,N] (True = present), weight [C,2H], bias [2H],
    norm_scale/norm_bias [C], out_weight [2H,D], out_bias [D],
    output_scale/output_bias [D] (used when output_norm). Parameters are
    stored [in][out] (the worked example fixes this orientation).
    Steps: sanitise absent tokens to zero; affine population LayerNorm;
    projection + bias; split the projected axis into q (first H) then k;
    pair (i, j) = [k_i * q_j, q_j - k_i]; output = pair @ out_weight +
    out_bias, then the optional affine LayerNorm; both tensors are zero
    unless tokens i and j are both present.
    `rows` (optional index array) restricts the result to query rows i."""
    x = _f64(x)
    m = _bool(mask)
    x = np.where(m[..., None], x, 0.0)
    y = layer_norm(x, eps, _f64(norm_scale), _f64(norm_bias)) @ _f64(weight) + _f64(bias)
    H = y.shape[-1] // 2
    q, k = y[..., :H], y[..., H:]
    N = x.shape[1]
    I = np.arange(N) if rows is None else np.asarray(rows)
    ki = k[:, I, None, :]            # [B, |I|, 1, H]
    qj = q[:, None, :, :]            # [B, 1, N, H]
    pf = np.concatenate([ki * qj, qj - ki], axis=-1)
    out = pf @ _f64(out_weight) + _f64(out_bias)
    if output_norm:
        out = layer_norm(out, eps, _f64(output_scale), _f64(output_bias))
    both = m[:, I, None] & m[:, None, :]
    pf = np.where(both[..., None], pf, 0.0)
    out = np.where(both[..., None], out, 0.0)
    return pf, out


def tied_row_attention(features, bias_features, norm_scale, norm_bias, bias_norm_scale,
                       bias_norm_bias, w_q, w_k, w_v, w_bias, w_gate, w_out, b_out,
                       eps=1e-5, heads=None):
    """[TIED]: the gated, projected update [B,L,L,C] (no residual added).

    features [B,L,L,C], bias_features [B,L,L,Cb]; norm_scale/norm_bias [C],
    bias_norm_scale/bias_norm_bias [Cb]; w_q, w_k, w_v, w_gate [C,H*D]
    (bias-free); w_bias [Cb,H]; w_out [H*D,C], b_out [C].
    Steps: exchange both pair axes of features and bias_features (X[s, i] =
    features[i, s]); affine LayerNorm of each over its channels; q, k, v,
    gate = sigmoid(. @ w_gate) and the per-head bias beta from them;
      A[i, j, h] = softmax_j( sum_{s,d} q[s,i,h,d] k[s,j,h,d] / sqrt(S*D)
                              + beta[i, j, h] )      (S = the tied axis length)
      U[i, k, h, d] = sum_j A[i, j, h] v[k, j, h, d]  (query i before anchor k)
    gated at (i, k) by the gate of X[i, k], projected over (h, d) with
    w_out and b_out, and the two axes exchanged back."""
    X = np.swapaxes(_f64(features), 1, 2)          # [B, S, L, C]
    Bf = np.swapaxes(_f64(bias_features), 1, 2)    # [B, L, L, Cb]
    xn = layer_norm(X, eps, _f64(norm_scale), _f64(norm_bias))
    bn = layer_norm(Bf, eps, _f64(bias_norm_scale), _f64(bias_norm_bias))
    wb = _f64(w_bias)
    H = wb.shape[-1] if heads is None else heads
    HD = _f64(w_q).shape[-1]
    D = HD // H
    B, S, L, _ = X.shape
    q = (xn @ _f64(w_q)).reshape(B, S, L, H, D)
    k = (xn @ _f64(w_k)).reshape(B, S, L, H, D)
    v = (xn @ _f64(w_v)).reshape(B, S, L, H, D)
    g = sigmoid(xn @ _f64(w_gate)).reshape(B, S, L, H, D)
    beta = bn @ wb                                  # [B, i, j, H]
    logits = np.einsum("bsihd,bsjhd->bhij", q, k) / np.sqrt(S * D)
    logits = logits + np.transpose(beta, (0, 3, 1, 2))
    logits = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(logits)
    A = e / e.sum(axis=-1, keepdims=True)           # [B, H, i, j]
    U = np.einsum("bhij,bkjhd->bikhd", A, v)        # [B, i, k, H, D]
    Ug = g * U                                      # gate of X at (i, k)
    out_t = Ug.reshape(B, S, L, HD) @ _f64(w_out) + _f64(b_out)
    return np.swapaxes(out_t, 1, 2)


def window_table(B, A, K, block=32, radius=-1):
    """[WIN]: key ids [B,A,K] of the windowed slot table: block b0 =
    block*floor(a/block) sees ids b0 - (K-block)//2 + k, k in [0, K). Ids
    outside [0, A) and, for radius >= 0, ids farther than radius from a are
    written as -1 (both are missing slots for the block)."""
    a = np.arange(A, dtype=np.int64)
    start = (a // block) * block - (K - block) // 2
    ids = start[:, None] + np.arange(K, dtype=np.int64)[None, :]
    bad = (ids < 0) | (ids >= A)
    if radius >= 0:
        bad |= np.abs(ids - a[:, None]) > radius
    ids = np.where(bad, -1, ids)
    return np.broadcast_to(ids, (B, A, K)).copy()
