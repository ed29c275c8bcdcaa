"""Seeded synthetic workloads for the windowed atom-attention block.

This module only draws inputs; it holds none of the block's arithmetic. The
tests feed the same tensors to the HIP path and to the fp64 oracle, and the
benchmark times the HIP path on them.

Recipes (the pages publish no dataset; their only workloads are two-atom
worked examples, so these synthetic inputs stand in for real molecules):

* matrices and biases ~ N(0, 0.1); ``*_scale`` vectors ~ 1 + N(0, 0.1);
  ``w_mod`` ~ N(0, 0.02); activations (atom, condition, pair, token) ~ N(0, 1);
* draws are fp32, rounded to bf16 (round-to-nearest-even) for bf16 workloads;
* rotary tables: angles ~ U(0, 2*pi) over D/2 frequencies, duplicated to the
  full width as [cos, cos] / [sin, sin]; with ``rope="distinct"`` the two
  halves come from independent angle draws, so a kernel that reads only one
  half of the supplied tables gives a different result;
* the window table W(32, K): a 32-query block starting at atom 32*floor(a/32)
  sees K consecutive atom ids centred on it, key_index[a, k] =
  32*floor(a/32) - (K-32)/2 + k; ids outside [0, A) stay in place and are
  therefore missing slots;
* unusable atoms carry NaN or +-Inf payloads (atom, condition and, for AF3,
  their pair rows), which the block must never read into arithmetic.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = ["Workload", "CONFIGS", "make_workload", "window_table", "make_s2p_workload",
           "make_tied_workload"]


@dataclasses.dataclass
class Workload:
    name: str
    style: str
    stage: str
    dtype: torch.dtype
    eps: float
    radius: int
    dims: Dict[str, int]
    activations: Dict[str, torch.Tensor]
    parameters: Dict[str, torch.Tensor]
    masks: Dict[str, torch.Tensor]
    structure: Dict[str, torch.Tensor]

    @property
    def entries(self) -> int:
        d = self.dims
        return d["B"] * d["A"] * d["H"] * d["K"]

    @property
    def atoms(self) -> int:
        return self.dims["B"] * self.dims["A"]

    def to(self, device) -> "Workload":
        mv = lambda d: {k: v.to(device) for k, v in d.items()}
        return dataclasses.replace(self, activations=mv(self.activations),
                                   parameters=mv(self.parameters),
                                   masks=mv(self.masks),
                                   structure=mv(self.structure))

    def kwargs(self):
        return dict(activations=self.activations, parameters=self.parameters,
                    masks=self.masks, structure=self.structure, eps=self.eps,
                    style=self.style, stage=self.stage, radius=self.radius)


# name -> recipe. "tokens" is the atom->token layout, "slots" the slot table
# recipe, "bad" the unusable-atom recipe.
CONFIGS = {
    # tiny AF3 encoder, fp32
    "0": dict(style="af3", stage="encoder", dtype=torch.float32, B=1, A=64,
              T=8, K=16, C=32, S=32, V=8, H=2, D=16, M=64, U=32, radius=-1,
              tokens="even", slots="random", bad="tiny", seed=0),
    # AF3 encoder, fp32
    "1": dict(style="af3", stage="encoder", dtype=torch.float32, B=1, A=4608,
              T=384, K=128, C=128, S=128, V=16, H=4, D=32, M=256, U=384,
              radius=-1, tokens="even", slots="window", bad="inf5", seed=1),
    # ESMFold2 encoder, bf16 storage, radius 48, 3% duplicated / 5% missing slots
    "2": dict(style="esmfold2", stage="encoder", dtype=torch.bfloat16, B=1,
              A=4608, T=384, K=128, C=128, S=128, V=16, H=4, D=32, M=256,
              U=384, radius=48, tokens="even", slots="window_dup3_miss5",
              bad="inf5", seed=2),
    # AF3 decoder, bf16, 4-20 atoms per token
    "3": dict(style="af3", stage="decoder", dtype=torch.bfloat16, B=4,
              A=12288, T=1024, K=128, C=128, S=128, V=16, H=4, D=32, M=256,
              U=384, radius=-1, tokens="variable", slots="window", bad="inf5",
              seed=3),
    # large mixed stress run, AF3 encoder, bf16
    "4a": dict(style="af3", stage="encoder", dtype=torch.bfloat16, B=1,
               A=24576, T=2048, K=128, C=128, S=128, V=16, H=4, D=32, M=256,
               U=384, radius=-1, tokens="even", slots="window_miss10_dup5",
               bad="mixed8", seed=4),
    # large mixed stress run, ESMFold2 encoder, bf16, radius 64
    "4b": dict(style="esmfold2", stage="encoder", dtype=torch.bfloat16, B=1,
               A=24576, T=2048, K=128, C=128, S=128, V=16, H=4, D=32, M=256,
               U=384, radius=64, tokens="even", slots="window_miss10_dup5",
               bad="mixed8", seed=5),
    # scattered key tables (ids uniform over the batch, 2 missing per row,
    # window_mask Bernoulli(0.9)) at the sizes of workloads 1 and 4a
    "1r": dict(style="af3", stage="encoder", dtype=torch.float32, B=1, A=4608,
               T=384, K=128, C=128, S=128, V=16, H=4, D=32, M=256, U=384,
               radius=-1, tokens="even", slots="random", bad="inf5", seed=11),
    "4r": dict(style="af3", stage="encoder", dtype=torch.bfloat16, B=1,
               A=24576, T=2048, K=128, C=128, S=128, V=16, H=4, D=32, M=256,
               U=384, radius=-1, tokens="even", slots="random", bad="mixed8",
               seed=14),
}


def window_table(B: int, A: int, K: int) -> torch.Tensor:
    """W(32, K): key_index[b, a, k] = 32*floor(a/32) - (K-32)//2 + k."""
    a = torch.arange(A, dtype=torch.int64)
    start = (a // 32) * 32 - (K - 32) // 2
    ki = start[:, None] + torch.arange(K, dtype=torch.int64)[None, :]
    return ki.unsqueeze(0).expand(B, A, K).contiguous()


def _perturb_slots(ki, g, dup_frac, miss_frac, miss_first):
    """Replace a fraction of slots by a copy of another slot's id in the same
    row (duplicates) and a fraction by -1 (missing)."""
    B, A, K = ki.shape
    ki = ki.clone()

    def dup():
        m = torch.rand((B, A, K), generator=g) < dup_frac
        src = torch.randint(0, K, (B, A, K), generator=g)
        ki[m] = torch.gather(ki, 2, src)[m]

    def miss():
        m = torch.rand((B, A, K), generator=g) < miss_frac
        ki[m] = -1

    if miss_first:
        miss(); dup()
    else:
        dup(); miss()
    return ki


def _variable_tokens(A, T, g):
    """Token sizes ~ U{4..20}, nudged by +-1 on random tokens (staying in
    [4, 20]) until they sum to A; atoms are assigned in sorted order."""
    lo, hi = 4, 20
    T = max(1, min(T, A // lo)) if A >= lo else 1
    while T * hi < A:
        T += 1
    sizes = torch.randint(lo, hi + 1, (T,), generator=g)
    diff = int(A - sizes.sum())
    while diff != 0:
        i = int(torch.randint(0, T, (1,), generator=g))
        if diff > 0 and sizes[i] < hi:
            sizes[i] += 1
            diff -= 1
        elif diff < 0 and sizes[i] > lo:
            sizes[i] -= 1
            diff += 1
    return T, torch.repeat_interleave(torch.arange(T, dtype=torch.int64), sizes)


def make_workload(name: str, seed: Optional[int] = None, A: Optional[int] = None,
                  B: Optional[int] = None, T: Optional[int] = None,
                  K: Optional[int] = None, dtype: Optional[torch.dtype] = None,
                  style: Optional[str] = None, stage: Optional[str] = None,
                  radius: Optional[int] = None, eps: float = 1e-5,
                  rope: str = "same", **widths: int) -> Workload:
    """Draw the named workload (optionally resized: A/B/T/K overrides keep the
    recipe, so a small instance spans a few tiles and a ragged tail; `widths`
    may override C, S, V, H, D, M, U). `rope` ("same" or "distinct") picks
    the rotary-table recipe of ESMFold2 workloads."""
    if rope not in ("same", "distinct"):
        raise ValueError("rope must be 'same' or 'distinct'")
    r = dict(CONFIGS[name])
    for k, v in widths.items():
        if k not in ("C", "S", "V", "H", "D", "M", "U"):
            raise TypeError("unknown width %r" % k)
        r[k] = int(v)
    if A is not None:
        r["A"] = A
        if T is None:
            T = max(1, (A * r["T"]) // CONFIGS[name]["A"])
    if T is not None:
        r["T"] = T
    if B is not None:
        r["B"] = B
    if K is not None:
        r["K"] = K
    if dtype is not None:
        r["dtype"] = dtype
    if style is not None:
        r["style"] = style
    if stage is not None:
        r["stage"] = stage
    if radius is not None:
        r["radius"] = radius
    seed = r["seed"] if seed is None else seed
    g = torch.Generator().manual_seed(seed)
    Bn, An, Tn, Kn = r["B"], r["A"], r["T"], r["K"]
    C, S, V, H, D, M, U = (r[k] for k in "C S V H D M U".split())
    HD = H * D
    style_, stage_ = r["style"], r["stage"]
    f32 = torch.float32

    def randn(*shape, std=1.0):
        return torch.randn(shape, generator=g, dtype=f32) * std

    # --- structure -----------------------------------------------------
    if r["tokens"] == "variable":
        rows = []
        Tn_eff = None
        for _ in range(Bn):
            t_b, a2t_b = _variable_tokens(An, Tn, g)
            Tn_eff = t_b if Tn_eff is None else max(Tn_eff, t_b)
            rows.append(a2t_b)
        Tn = Tn_eff
        a2t = torch.stack(rows)
    else:
        per = max(1, An // Tn)
        a2t = (torch.arange(An, dtype=torch.int64) // per).clamp(max=Tn - 1)
        a2t = a2t.unsqueeze(0).expand(Bn, An).contiguous()

    if r["slots"] == "random":
        ki = torch.randint(0, An, (Bn, An, Kn), generator=g)
        nmiss = min(2, Kn)
        for b in range(Bn):
            for a in range(An):
                pos = torch.randperm(Kn, generator=g)[:nmiss]
                ki[b, a, pos] = -1
        wm = torch.rand((Bn, An, Kn), generator=g) < 0.9
    else:
        ki = window_table(Bn, An, Kn)
        if r["slots"] == "window_dup3_miss5":
            ki = _perturb_slots(ki, g, 0.03, 0.05, miss_first=False)
        elif r["slots"] == "window_miss10_dup5":
            ki = _perturb_slots(ki, g, 0.05, 0.10, miss_first=True)
        wm = torch.ones((Bn, An, Kn), dtype=torch.bool)

    valid = torch.ones((Bn, An), dtype=torch.bool)
    token_valid = torch.ones((Bn, Tn), dtype=torch.bool)
    bad = r["bad"]
    if bad == "tiny":
        nbad = max(1, round(0.1 * An))
        for b in range(Bn):
            valid[b, torch.randperm(An, generator=g)[:nbad]] = False
    elif bad == "inf5":
        nbad = max(1, round(0.05 * An))
        for b in range(Bn):
            valid[b, torch.randperm(An, generator=g)[:nbad]] = False
    elif bad == "mixed8":
        n_inv = max(1, round(0.04 * An))
        n_oor = max(1, round(0.02 * An))
        n_tok = max(1, round(0.02 * An / max(1, An // Tn)))
        for b in range(Bn):
            perm = torch.randperm(An, generator=g)
            valid[b, perm[:n_inv]] = False
            oor = perm[n_inv:n_inv + n_oor]
            flip = torch.rand(len(oor), generator=g) < 0.5
            a2t[b, oor] = torch.where(flip, torch.full_like(oor, -1),
                                      torch.full_like(oor, Tn))
            token_valid[b, torch.randperm(Tn, generator=g)[:n_tok]] = False

    in_range = (a2t >= 0) & (a2t < Tn)
    tv_of_atom = torch.gather(token_valid, 1, a2t.clamp(0, Tn - 1))
    unusable = ~(valid & in_range & tv_of_atom)

    # --- activations ---------------------------------------------------
    atom = randn(Bn, An, C)
    cond = randn(Bn, An, S)
    acts = {}
    if bad in ("inf5",):
        sign = torch.where(torch.rand((Bn, An, 1), generator=g) < 0.5, -1.0, 1.0)
        junk = sign * math.inf
    else:
        junk = torch.full((Bn, An, 1), math.nan)
    atom = torch.where(unusable[..., None], junk.expand_as(atom), atom)
    cond = torch.where(unusable[..., None], junk[..., :1].expand_as(cond), cond)
    acts["atom"] = atom
    acts["condition"] = cond
    if style_ == "af3":
        pair = randn(Bn, An, Kn, V)
        pj = junk[..., None].expand(Bn, An, Kn, V)
        pair = torch.where(unusable[..., None, None], pj, pair)
        if bad == "mixed8":
            # inactive pair rows of missing slots carry NaN as well
            missing = (ki < 0) | (ki >= An)
            pair = torch.where(missing[..., None], torch.full_like(pair, math.nan), pair)
        acts["pair"] = pair
    else:
        theta = torch.rand((Bn, An, D // 2), generator=g, dtype=f32) * (2 * math.pi)
        theta2 = theta
        if rope == "distinct":
            theta2 = torch.rand((Bn, An, D // 2), generator=g, dtype=f32) * (2 * math.pi)
        acts["rope_cos"] = torch.cat([theta.cos(), theta2.cos()], dim=-1)
        acts["rope_sin"] = torch.cat([theta.sin(), theta2.sin()], dim=-1)
    if stage_ == "decoder":
        tok = randn(Bn, Tn, U)
        tok = torch.where(token_valid[..., None], tok, torch.full_like(tok, math.nan))
        acts["token"] = tok

    # --- parameters ----------------------------------------------------
    p = {}
    w = 0.1
    if style_ == "af3":
        p["cond_scale"] = 1.0 + randn(3, S, std=w)
        p["w_scale"] = randn(3, S, C, std=w)
        p["b_scale"] = randn(3, C, std=w)
        p["w_shift"] = randn(3, S, C, std=w)
        p["w_residual_gate"] = randn(2, S, C, std=w)
        p["b_residual_gate"] = randn(2, C, std=w)
    else:
        p["w_mod"] = randn(S, 6, C, std=0.02)
    p["w_q"] = randn(C, HD, std=w)
    if style_ == "af3":
        p["b_q"] = randn(HD, std=w)
    p["w_k"] = randn(C, HD, std=w)
    p["w_v"] = randn(C, HD, std=w)
    if style_ == "af3":
        p["pair_scale"] = 1.0 + randn(V, std=w)
        p["w_pair"] = randn(V, H, std=w)
    p["w_value_gate"] = randn(C, HD, std=w)
    p["w_attention_out"] = randn(HD, C, std=w)
    p["w_ff_gate"] = randn(C, M, std=w)
    p["w_ff_up"] = randn(C, M, std=w)
    p["w_ff_out"] = randn(M, C, std=w)
    if stage_ == "encoder":
        p["w_pool"] = randn(C, U, std=w)
    else:
        p["w_token"] = randn(U, C, std=w)
        p["readout_scale"] = 1.0 + randn(C, std=w)
        if style_ == "esmfold2":
            p["readout_bias"] = randn(C, std=w)
        p["w_readout"] = randn(C, 3, std=w)

    dt = r["dtype"]
    acts = {k: v.to(dt).contiguous() for k, v in acts.items()}
    p = {k: v.to(dt).contiguous() for k, v in p.items()}
    masks = {"valid": valid.contiguous(), "token_valid": token_valid.contiguous(),
             "window_mask": wm.contiguous()}
    structure = {"atom_to_token": a2t.contiguous(), "key_index": ki.contiguous()}
    dims = dict(B=Bn, A=An, T=Tn, K=Kn, C=C, S=S, H=H, D=D,
                V=V if style_ == "af3" else 1, M=M, U=U)
    return Workload(name=name, style=style_, stage=stage_, dtype=dt, eps=eps,
                    radius=r["radius"], dims=dims, activations=acts,
                    parameters=p, masks=masks, structure=structure)


def make_s2p_workload(B: int = 1, N: int = 512, C: int = 1024, H: int = 64, D: int = 128,
                      dtype: torch.dtype = torch.bfloat16, seed: int = 7,
                      absent: float = 0.05, output_norm: bool = False):
    """Inputs of the single-to-pair operator (the pages give no workload; the
    default sizes are an ESMFold-like trunk: 1024-wide token states, q and k
    of width 64, a 128-wide pair head, 512 tokens). x ~ N(0, 1), matrices
    ~ N(0, 1/sqrt(fan_in)), biases ~ N(0, 0.1), norm scales ~ 1 + N(0, 0.1);
    a fraction `absent` of tokens is absent with NaN payloads. Returns
    (activations, parameters, masks, output_norm) for the page's signature."""
    g = torch.Generator().manual_seed(seed)
    f32 = torch.float32

    def randn(*shape, std=1.0, mean=0.0):
        return torch.randn(shape, generator=g, dtype=f32) * std + mean

    x = randn(B, N, C)
    mask = torch.rand((B, N), generator=g) >= absent
    x = torch.where(mask[..., None], x, torch.full_like(x, math.nan))
    p = {"weight": randn(C, 2 * H, std=1.0 / math.sqrt(C)), "bias": randn(2 * H, std=0.1),
         "norm_scale": randn(C, std=0.1, mean=1.0), "norm_bias": randn(C, std=0.1),
         "out_weight": randn(2 * H, D, std=1.0 / math.sqrt(2 * H)), "out_bias": randn(D, std=0.1),
         "output_scale": randn(D, std=0.1, mean=1.0), "output_bias": randn(D, std=0.1)}
    acts = {"x": x.to(dtype).contiguous()}
    p = {k: v.to(dtype).contiguous() for k, v in p.items()}
    return acts, p, {"mask": mask.contiguous()}, output_norm


def make_tied_workload(B: int = 1, L: int = 256, C: int = 128, CB: int = 128, H: int = 4,
                       D: int = 32, dtype: torch.dtype = torch.bfloat16, seed: int = 9):
    """Inputs of tied pair row attention (the pages give no workload; the
    default sizes are a pair stack of a 256-residue crop: 128 pair channels,
    4 heads of width 32, 128-wide bias features). features and
    bias_features ~ N(0, 1); matrices ~ N(0, 1/sqrt(fan_in)); norm scales
    ~ 1 + N(0, 0.1), shifts and b_out ~ N(0, 0.1). Returns (activations,
    parameters) for the page's signature."""
    g = torch.Generator().manual_seed(seed)
    f32 = torch.float32

    def randn(*shape, std=1.0, mean=0.0):
        return torch.randn(shape, generator=g, dtype=f32) * std + mean

    HD = H * D
    acts = {"features": randn(B, L, L, C), "bias_features": randn(B, L, L, CB)}
    p = {"norm_scale": randn(C, std=0.1, mean=1.0), "norm_bias": randn(C, std=0.1),
         "bias_norm_scale": randn(CB, std=0.1, mean=1.0), "bias_norm_bias": randn(CB, std=0.1),
         "w_q": randn(C, HD, std=C ** -0.5), "w_k": randn(C, HD, std=C ** -0.5),
         "w_v": randn(C, HD, std=C ** -0.5), "w_bias": randn(CB, H, std=CB ** -0.5),
         "w_gate": randn(C, HD, std=C ** -0.5), "w_out": randn(HD, C, std=HD ** -0.5),
         "b_out": randn(C, std=0.1)}
    acts = {k: v.to(dtype).contiguous() for k, v in acts.items()}
    p = {k: v.to(dtype).contiguous() for k, v in p.items()}
    return acts, p
