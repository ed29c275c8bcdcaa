"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs.

* small instances of every workload recipe (a few tiles plus a ragged tail),
  all outputs element by element;
* the full-size workloads in the launch configuration the benchmark times,
  on sampled atoms/tokens the oracle computes one by one, plus properties
  that hold at any size;
* masks bit-exact; the slot-attention step alone on seeded Q/K/V;
* invariants on the GPU path itself (junk payloads, radius, batches,
  determinism), the subnormal sigmoid tail and the pooling precondition
  status word.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from _parity import (RTOL, assert_close, assert_close_rel, compare_block, exact_zero_checks,
                     np64, run_gpu)
from windowed_atom_attention_amd import masks as gpu_masks
from windowed_atom_attention_amd import slot_attention as gpu_slot_attention
from windowed_atom_attention_amd import pack_params, windowed_atom_attention, workspace_bytes
from windowed_atom_attention_amd.workloads import make_workload

pytestmark = pytest.mark.gpu

SMALL = [
    ("0", {}),
    ("1", dict(A=300)),
    ("2", dict(A=300)),
    ("3", dict(B=2, A=400)),
    ("4a", dict(A=500)),
    ("4b", dict(A=500)),
    # the other style/stage/dtype combinations on the same recipes
    ("0", dict(stage="decoder")),
    ("0", dict(style="esmfold2")),
    ("0", dict(style="esmfold2", stage="decoder", dtype=torch.bfloat16)),
    ("1", dict(A=200, dtype=torch.bfloat16)),
    ("2", dict(A=200, dtype=torch.float32, stage="decoder")),
    ("3", dict(B=2, A=300, dtype=torch.float32, style="esmfold2")),
    ("4a", dict(A=333, stage="decoder", radius=20)),
    # random key ids over hundreds of atoms: key bands wider than one chunk
    ("0", dict(A=600)),
    ("0", dict(A=450, K=40, style="esmfold2", dtype=torch.bfloat16)),
    ("0", dict(A=300, K=200, dtype=torch.bfloat16, stage="decoder")),
    # bf16 rows that are not whole 16-byte vectors (attention stored per value)
    ("0", dict(A=200, K=45, dtype=torch.bfloat16)),
    ("0", dict(A=200, K=21, style="esmfold2", dtype=torch.bfloat16)),
    # every pair-row width the slot kernel specialises on (AF3 bf16: 8, 16,
    # 24, 32 channels; fp32: 8, 16), and wider heads
    ("0", dict(A=200, V=24, K=64, dtype=torch.bfloat16)),
    ("0", dict(A=200, V=32, dtype=torch.bfloat16, K=40)),
    ("0", dict(A=150, V=16, H=4, D=64)),
    ("0", dict(A=150, H=2, D=128, V=16, dtype=torch.bfloat16, stage="decoder")),
    ("0", dict(A=200, K=48, style="esmfold2", H=8, D=16)),
    # more 32-atom tiles than compute units: the projection kernels' 4-wave
    # form (small grids take the 8-wave form that splits k over wave pairs)
    ("0", dict(B=30, A=300)),
    ("0", dict(B=30, A=300, style="esmfold2", stage="decoder", dtype=torch.bfloat16)),
    # rotary tables whose two halves differ (the full-width tables are used
    # as supplied)
    ("2", dict(A=300, rope="distinct")),
    ("4b", dict(A=400, rope="distinct", dtype=torch.float32, stage="decoder")),
    # scattered key ids over thousands of atoms: query blocks whose key band
    # spans more than eight 128-row chunks are computed by the gather kernel
    ("0", dict(A=2000, K=64)),
    ("0", dict(A=1500, K=48, style="esmfold2", dtype=torch.bfloat16, stage="decoder")),
    ("0", dict(A=2500, K=40, dtype=torch.bfloat16)),   # AF3 pair bias precomputed
    ("0", dict(A=9000, K=24, dtype=torch.bfloat16)),   # AF3 pair bias from the pair rows
    ("0", dict(A=2000, K=32, H=2, D=128, V=16, dtype=torch.bfloat16)),
    ("0", dict(A=2100, K=20, style="esmfold2", H=8, D=16)),
]


def _id(case):
    name, kw = case
    return name + "-" + "-".join("%s=%s" % (k, str(v).replace("torch.", "")) for k, v in kw.items())


@pytest.mark.parametrize("case", SMALL, ids=[_id(c) for c in SMALL])
def test_block_small_matches_oracle(case):
    name, kw = case
    w = make_workload(name, **kw)
    print("case", _id(case), w.dims, flush=True)
    gpu = run_gpu(w)
    ref = oracle.block(**w.kwargs(), intermediates=True)
    exact_zero_checks(w, gpu, ref["usable"], ref["allowed"])
    compare_block(w, gpu, ref)


@pytest.mark.parametrize("name", ["0", "2", "3", "4a", "4b"])
def test_masks_bit_exact(name):
    w = make_workload(name, A=None if name == "0" else 700, B=2 if name == "3" else None)
    g = w.to("cuda")
    us, al, cnt = gpu_masks(g.masks, g.structure, w.dims["T"], w.radius)
    ref = oracle.block(**w.kwargs(), intermediates=True)
    assert np.array_equal(us.cpu().numpy(), ref["usable"].astype(bool))
    assert np.array_equal(al.cpu().numpy(), ref["allowed"].astype(bool))
    # usable atoms per token, counted on the host from the oracle's mask
    B, T = w.dims["B"], w.dims["T"]
    exp = np.zeros((B, T), np.int64)
    a2t = w.structure["atom_to_token"].numpy()
    u = ref["usable"].astype(bool)
    for b in range(B):
        np.add.at(exp[b], a2t[b][u[b]], 1)
    assert np.array_equal(cnt.cpu().numpy().astype(np.int64), exp)


@pytest.mark.parametrize("style", ["af3", "esmfold2"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_slot_attention_step(style, dtype):
    w = make_workload("4a" if style == "af3" else "4b", A=600, dtype=dtype)
    ref_masks = oracle.block(**w.kwargs(), intermediates=True)
    B, A = w.dims["B"], w.dims["A"]
    HD = w.dims["H"] * w.dims["D"]
    gen = torch.Generator().manual_seed(17)
    q, k, v = (torch.randn((B, A, HD), generator=gen).to(dtype) for _ in range(3))
    usable = torch.from_numpy(ref_masks["usable"]).bool()
    # payloads of unusable atoms are junk (NaN and +-Inf) and must not leak
    bad = ~usable
    junk = torch.tensor([float("nan"), float("inf"), -float("inf")], dtype=dtype)
    for t in (q, k, v):
        t[bad] = junk[torch.arange(int(bad.sum())) % 3][:, None].expand(-1, HD)
    kw = dict(eps=w.eps, style=style, radius=w.radius)
    pair = pair_scale = w_pair = None
    if style == "af3":
        pair = w.activations["pair"]
        pair_scale = w.parameters["pair_scale"]
        w_pair = w.parameters["w_pair"]
    ref = oracle.slot_attention(q, k, v, usable, w.structure["key_index"],
                                w.masks["window_mask"], heads=w.dims["H"],
                                pair=pair, pair_scale=pair_scale, w_pair=w_pair, **kw)
    cu = lambda t: None if t is None else t.cuda()
    att, o = gpu_slot_attention(cu(q), cu(k), cu(v), cu(usable), cu(w.structure["key_index"]),
                                cu(w.masks["window_mask"]), heads=w.dims["H"],
                                pair=cu(pair), pair_scale=cu(pair_scale), w_pair=cu(w_pair), **kw)
    rtol = RTOL[dtype]
    al = ref["allowed"].astype(bool)
    attn = np64(att)
    assert np.all(attn[np.broadcast_to(~al[:, None], attn.shape)] == 0.0)
    assert_close_rel("attention", attn, ref["attention"], rtol)
    assert np.all(np.isfinite(np64(o)))
    assert_close("o", np64(o), ref["o"], rtol)
    assert np.all(np64(o)[~ref_masks["usable"].astype(bool)] == 0.0)


PREPACKED = [
    ("1", dict(A=700)),                     # one tile per CU at most: strip layout
    ("0", dict(B=30, A=300)),               # more tiles than CUs: 32-column blocks
    ("3", dict(B=2, A=600)),                # decoder: w_token stays in block layout
    ("4b", dict(A=900, stage="decoder")),
    ("2", dict(A=400, dtype=torch.float32)),
]


@pytest.mark.parametrize("case", PREPACKED, ids=[_id(c) for c in PREPACKED])
def test_prepacked_weights_equal_per_call_packing(case):
    """Weights packed once (atom_attn_pack_params) give the same bits as the
    call that packs them itself, for both projection-kernel forms; one
    packed buffer serves calls of different grid sizes."""
    name, kw = case
    w = make_workload(name, **kw)
    print("prepacked", _id(case), w.dims, flush=True)
    g = w.to("cuda")
    ref = windowed_atom_attention(**g.kwargs())
    pk = pack_params(g.parameters, w.dims, w.style, w.stage)
    got = windowed_atom_attention(**g.kwargs(), packed=pk)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k].view(torch.uint8), ref[k].view(torch.uint8)), k
    # the same packed weights on a smaller grid of the same widths
    w2 = make_workload(name, **dict(kw, A=max(64, kw.get("A", 64) // 3), B=1))
    g2 = w2.to("cuda")
    g2 = dataclasses.replace(g2, parameters=g.parameters)
    ref2 = windowed_atom_attention(**g2.kwargs())
    got2 = windowed_atom_attention(**g2.kwargs(), packed=pk)
    torch.cuda.synchronize()
    for k in ref2:
        assert torch.equal(got2[k].view(torch.uint8), ref2[k].view(torch.uint8)), k


# ------------------------------------------------------- full size, sampled

FULL = ["1", "2", "3", "4a", "4b"]


def _sample_rows(w, n=48, seed=0):
    B, A = w.dims["B"], w.dims["A"]
    g = np.random.default_rng(seed)
    sel = np.zeros((B, A), bool)
    for b in range(B):
        # first/last atoms, tile and block boundaries, and random atoms
        fixed = [0, 1, 15, 16, 31, 32, A // 2, A - 33, A - 32, A - 17, A - 16, A - 1]
        sel[b, [a for a in fixed if 0 <= a < A]] = True
        sel[b, g.integers(0, A, n // B)] = True
    return sel


@pytest.mark.parametrize("name", FULL)
def test_block_full_size_sampled(name):
    w = make_workload(name)
    print("full", name, w.dims, flush=True)
    gpu = run_gpu(w)
    sel = _sample_rows(w)
    ref = oracle.block(**w.kwargs(), select=torch.from_numpy(sel), intermediates=False)
    rows = ref["done_atom"].astype(bool)
    toks = ref["done_token"].astype(bool) if w.stage == "encoder" else None
    assert rows[sel].all()
    compare_block(w, gpu, ref, rows=rows, tokens=toks)
    # properties at full size: finite outputs, attention rows sum to 1 or 0
    for k, v in gpu.items():
        assert torch.isfinite(v.float()).all(), k
    rs = gpu["attention"].float().sum(-1)
    tol = 1e-4 if w.dtype == torch.float32 else 3e-2
    assert bool(((rs - 1).abs() < tol).logical_or(rs == 0).all())
    g = w.to("cuda")
    us, al, _ = gpu_masks(g.masks, g.structure, w.dims["T"], w.radius)
    empty = ~al.any(-1)  # rows without allowed slots: exactly zero
    assert bool((rs.transpose(0, 1)[:, empty] == 0).all())
    assert bool((gpu["hidden"][~us] == 0).all())


# --------------------------------------------------------- invariants

@pytest.mark.parametrize("name,kw", [("0", {}), ("4a", dict(A=400)),
                                     ("4b", dict(A=400)), ("3", dict(B=2, A=300))])
def test_junk_payloads_do_not_leak_bitwise(name, kw):
    w = make_workload(name, **kw)
    r1 = run_gpu(w)
    ref = oracle.block(**w.kwargs(), intermediates=True)
    us = torch.from_numpy(ref["usable"]).bool()
    al = torch.from_numpy(ref["allowed"]).bool()
    w2 = make_workload(name, **kw)
    for k in ("atom", "condition"):
        w2.activations[k][~us] = 0.0
    if "pair" in w2.activations:
        w2.activations["pair"][~al] = 0.0
    if "token" in w2.activations:
        tv = w2.masks["token_valid"]
        w2.activations["token"][~tv] = 0.0
    r2 = run_gpu(w2)
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k


@pytest.mark.parametrize("name", ["0", "4b"])
def test_radius_minus_one_equals_unlimited_bitwise(name):
    w = make_workload(name, A=None if name == "0" else 300)
    w.radius = -1
    r1 = run_gpu(w)
    w.radius = w.dims["A"] - 1
    r2 = run_gpu(w)
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k


def test_batches_do_not_mix_bitwise():
    w = make_workload("3", B=3, A=256, dtype=torch.float32)
    r1 = run_gpu(w)
    w2 = make_workload("3", B=3, A=256, dtype=torch.float32)
    g = torch.Generator().manual_seed(5)
    for v in w2.activations.values():
        v[1] = torch.randn(v[1].shape, generator=g).to(v.dtype)
    r2 = run_gpu(w2)
    for k in r1:  # batch is axis 0 of every output
        assert torch.equal(r1[k][0], r2[k][0]), k
        assert torch.equal(r1[k][2], r2[k][2]), k
        assert not torch.equal(r1[k][1], r2[k][1]), k


@pytest.mark.parametrize("name", ["1", "4a"])
def test_deterministic_bitwise(name):
    w = make_workload(name, A=1000)
    r1 = run_gpu(w)
    r2 = run_gpu(w)
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k


def test_all_missing_windows_and_unusable_everything():
    w = make_workload("1", A=200)
    w.masks["window_mask"][:] = False
    gpu = run_gpu(w)
    ref = oracle.block(**w.kwargs(), intermediates=True)
    assert bool((gpu["attention"] == 0).all())
    compare_block(w, gpu, ref)
    w = make_workload("1", A=200)
    w.masks["valid"][:] = False
    gpu = run_gpu(w)
    for k, v in gpu.items():
        assert bool((v == 0).all()), k


def test_sigmoid_subnormal_tail_fp32():
    """AF3 attention gate sigmoid(-95) = 5.5e-42 is a subnormal fp32 value;
    with a zero entry state and zero transition output it is visible in
    hidden and must not be flushed."""
    w = make_workload("0", A=40)
    p = w.parameters
    p["w_residual_gate"].zero_()
    p["b_residual_gate"][0] = -95.0
    p["w_ff_out"].zero_()
    a = int(torch.nonzero(w.masks["valid"][0])[0])  # first usable atom
    w.activations["atom"][0, a] = 0.0
    gpu = run_gpu(w)
    ref = oracle.block(**w.kwargs())
    h = np64(gpu["hidden"])[0, a]
    r = ref["hidden"][0, a]
    big = np.abs(r) > 1e-43
    assert big.any()
    assert np.all(h[big] != 0.0)
    np.testing.assert_allclose(h[big], r[big], rtol=2e-2)


def test_status_word_reports_unsorted_tokens():
    w = make_workload("1", A=256)
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    g = w.to("cuda")
    windowed_atom_attention(**g.kwargs(), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    a2t = w.structure["atom_to_token"].clone()
    a2t[0, 100:112] = 1  # a token reappearing after later ones
    w.structure["atom_to_token"] = a2t
    g = w.to("cuda")
    out = windowed_atom_attention(**g.kwargs(), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    # the other outputs are unaffected by the precondition
    ref = oracle.block(**w.kwargs())
    assert_close("hidden", np64(out["hidden"]), ref["hidden"], RTOL[w.dtype])


def test_strided_inputs_are_not_mutated():
    w = make_workload("0")
    g = w.to("cuda")
    # a non-contiguous atom tensor with the same values
    big = torch.zeros((1, 64, 64), device="cuda")
    big[..., ::2] = g.activations["atom"]
    g.activations["atom"] = big[..., ::2]
    before = {k: v.clone() for k, v in g.activations.items()}
    out = windowed_atom_attention(**g.kwargs())
    torch.cuda.synchronize()
    for k, v in g.activations.items():
        assert torch.equal(v.nan_to_num(), before[k].nan_to_num()), k
    ref = oracle.block(**w.kwargs())
    assert_close("hidden", np64(out["hidden"]), ref["hidden"], RTOL[w.dtype])


def test_graph_capture_replays_match_eager():
    """One block call captured in a HIP graph: every replay, with eager work
    and synchronisations between replays, rewrites the outputs bit for bit as
    the eager call did (window slots without repeated key ids, whose weights
    would be summed in a run-dependent order)."""
    w = make_workload("1", A=700)
    g = w.to("cuda")
    ws = torch.empty(workspace_bytes(w.dims, w.style, w.stage, w.dtype),
                     dtype=torch.uint8, device="cuda")
    out = windowed_atom_attention(**g.kwargs(), workspace=ws)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        windowed_atom_attention(**g.kwargs(), workspace=ws, out=out)
    torch.cuda.synchronize()
    for _ in range(3):
        for v in out.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), k


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pooling_tokens_across_tiles(dtype):
    """Token layouts the tile-local pooling has to join: a token of 100
    atoms spanning four 32-atom tiles, with a whole tile of unusable atoms
    inside it; a token ending exactly at a tile boundary; one-atom tokens;
    a batch boundary inside a tile (B=2, A=150); empty tokens."""
    w = make_workload("1", B=2, A=150, dtype=dtype)
    B, A, T = w.dims["B"], w.dims["A"], w.dims["T"]
    a2t = torch.zeros((B, A), dtype=torch.int64)
    for b in range(B):
        pos, t = 0, 0
        for size in [100, 28, 1, 1, 5] + [3] * 10:
            if pos >= A or t >= T:
                break
            a2t[b, pos:pos + size] = t
            pos += size
            t += 2 if size == 1 else 1  # odd ids after one-atom tokens stay empty
        a2t[b, pos:] = min(t, T - 1)
    w.structure["atom_to_token"] = a2t
    valid = w.masks["valid"].clone()
    valid[0, 40:75] = False  # an unusable tile inside the long token
    w.masks["valid"] = valid
    tv = w.masks["token_valid"].clone()
    tv[:] = True
    w.masks["token_valid"] = tv
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    g = w.to("cuda")
    out = windowed_atom_attention(**g.kwargs(), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = oracle.block(**w.kwargs(), intermediates=True)
    assert_close("token_output", np64(out["token_output"]), ref["token_output"], RTOL[dtype])
    exact_zero_checks(w, {k: v for k, v in out.items()}, ref["usable"], ref["allowed"])


# ------------------------------------------------- device window table

@pytest.mark.parametrize("B,A,K,block,radius", [
    (1, 300, 128, 32, -1), (2, 1000, 128, 32, 48), (1, 97, 21, 8, 5),   # ragged rows
    (3, 50, 8, 16, 0), (1, 40, 5, 8, -1),                              # K < block, odd difference
    (4, 12288, 128, 32, -1),                                            # decoder workload size
])
def test_window_table_bit_exact(B, A, K, block, radius):
    from oracle import pair_ops
    from windowed_atom_attention_amd import window_table
    print("window", B, A, K, block, radius, flush=True)
    exp = pair_ops.window_table(B, A, K, block=block, radius=radius)
    for dt in (torch.int64, torch.int32):
        got = window_table(B, A, K, block=block, radius=radius, dtype=dt)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().astype(np.int64), exp), dt


def test_block_with_device_window_table_matches_host_table():
    """The block gives the same bits with the device-built table (missing
    ids written as -1, radius folded in) as with the generator's table."""
    from windowed_atom_attention_amd import window_table
    from windowed_atom_attention_amd.workloads import window_table as host_table
    w = make_workload("4b", A=700)
    w.structure["key_index"] = host_table(1, 700, 128)
    g = w.to("cuda")
    ref = windowed_atom_attention(**g.kwargs())
    g.structure["key_index"] = window_table(1, 700, 128, radius=w.radius)
    got = windowed_atom_attention(**g.kwargs())
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k].view(torch.uint8), ref[k].view(torch.uint8)), k


# ---------------------------------------------------- single-to-pair features

S2P_CASES = [
    dict(B=1, N=70, C=96, H=32, D=64, dtype=torch.float32, output_norm=False),
    dict(B=2, N=45, C=64, H=64, D=128, dtype=torch.float32, output_norm=True),
    dict(B=1, N=100, C=1024, H=64, D=128, dtype=torch.bfloat16, output_norm=False),
    dict(B=2, N=33, C=200, H=128, D=256, dtype=torch.bfloat16, output_norm=True),
    dict(B=1, N=64, C=128, H=32, D=128, dtype=torch.bfloat16, output_norm=True),
]


def _s2p_case_id(c):
    return "B%(B)d-N%(N)d-C%(C)d-H%(H)d-D%(D)d-" % c + ("bf16" if c["dtype"] == torch.bfloat16 else "f32") + \
        ("-norm" if c["output_norm"] else "")


def _s2p_check(acts, par, masks, on, pf, out, rows=None):
    from oracle import pair_ops
    rtol = RTOL[acts["x"].dtype]
    ref_pf, ref_out = pair_ops.single_to_pair(
        acts["x"], masks["mask"], par["weight"], par["bias"], par["norm_scale"],
        par["norm_bias"], par["out_weight"], par["out_bias"], eps=1e-5, output_norm=on,
        output_scale=par["output_scale"], output_bias=par["output_bias"], rows=rows)
    gpf, gout = np64(pf), np64(out)
    if rows is not None:
        gpf, gout = gpf[:, rows], gout[:, rows]
    m = masks["mask"].numpy()
    I = np.arange(m.shape[1]) if rows is None else rows
    both = m[:, I, None] & m[:, None, :]
    assert np.all(gpf[~both] == 0.0) and np.all(gout[~both] == 0.0)
    assert_close("pair_features", gpf, ref_pf, rtol)
    assert_close("output", gout, ref_out, rtol)


@pytest.mark.parametrize("case", S2P_CASES, ids=[_s2p_case_id(c) for c in S2P_CASES])
def test_single_to_pair_matches_oracle(case):
    from windowed_atom_attention_amd import single_to_pair
    from windowed_atom_attention_amd.workloads import make_s2p_workload
    c = dict(case)
    print("s2p", _s2p_case_id(c), flush=True)
    acts, par, masks, on = make_s2p_workload(**c, seed=11)
    cu = lambda d: {k: v.cuda() for k, v in d.items()}
    pf, out = single_to_pair(cu(acts), cu(par), cu(masks), output_norm=on)
    torch.cuda.synchronize()
    _s2p_check(acts, par, masks, on, pf, out)


def test_single_to_pair_full_size_sampled_rows():
    """The benchmarked size (B=1, N=512, C=1024, H=64, D=128, bf16) on
    sampled query rows the oracle computes alone, both output modes."""
    from windowed_atom_attention_amd import single_to_pair
    from windowed_atom_attention_amd.workloads import make_s2p_workload
    rows = np.array([0, 1, 31, 32, 255, 256, 480, 510, 511])
    for on in (False, True):
        acts, par, masks, _ = make_s2p_workload(output_norm=on)
        cu = lambda d: {k: v.cuda() for k, v in d.items()}
        pf, out = single_to_pair(cu(acts), cu(par), cu(masks), output_norm=on)
        torch.cuda.synchronize()
        assert torch.isfinite(pf.float()).all() and torch.isfinite(out.float()).all()
        _s2p_check(acts, par, masks, on, pf, out, rows=rows)


# ------------------------------------------------- tied pair row attention

TIED_CASES = [
    dict(B=1, L=37, C=64, CB=16, H=2, D=32, dtype=torch.float32),     # ragged grid
    dict(B=2, L=64, C=128, CB=32, H=4, D=32, dtype=torch.float32),
    dict(B=1, L=100, C=32, CB=8, H=1, D=32, dtype=torch.bfloat16),
    dict(B=2, L=45, C=96, CB=40, H=3, D=32, dtype=torch.bfloat16),
    dict(B=1, L=70, C=256, CB=128, H=8, D=32, dtype=torch.bfloat16),
    dict(B=1, L=40, C=64, CB=24, H=6, D=32, dtype=torch.float32),     # bias rows padded to 8 heads, any width
    dict(B=1, L=1, C=32, CB=4, H=1, D=32, dtype=torch.float32),       # one residue
]


def _tied_id(c):
    return "B%(B)d-L%(L)d-C%(C)d-CB%(CB)d-H%(H)d" % c + ("-bf16" if c["dtype"] == torch.bfloat16 else "-f32")


def _tied_check(acts, par, got, rtol):
    from oracle import pair_ops
    ref = pair_ops.tied_row_attention(
        acts["features"], acts["bias_features"], par["norm_scale"], par["norm_bias"],
        par["bias_norm_scale"], par["bias_norm_bias"], par["w_q"], par["w_k"], par["w_v"],
        par["w_bias"], par["w_gate"], par["w_out"], par["b_out"], eps=1e-5)
    g = np64(got)
    assert np.all(np.isfinite(g))
    assert_close("tied update", g, ref, rtol)


@pytest.mark.parametrize("case", TIED_CASES, ids=[_tied_id(c) for c in TIED_CASES])
def test_tied_row_attention_matches_oracle(case):
    from windowed_atom_attention_amd import tied_row_attention
    from windowed_atom_attention_amd.workloads import make_tied_workload
    print("tied", _tied_id(case), flush=True)
    acts, par = make_tied_workload(**case, seed=12)
    cu = lambda d: {k: v.cuda() for k, v in d.items()}
    got = tied_row_attention(cu(acts), cu(par))
    torch.cuda.synchronize()
    _tied_check(acts, par, got, RTOL[case["dtype"]])


def test_tied_row_attention_worked_example_on_gpu():
    """The page's worked example (fp32, L=2, C=2 padded to the kernel's
    supported widths with zero channels and weights) gives its closed form."""
    import json
    import math
    import os
    from windowed_atom_attention_amd import tied_row_attention
    g = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                    "tied_pair_row_attention_worked_example.json")))
    p_ = 1.0 / (1.0 + math.exp(-math.sqrt(2.0)))
    # C = 2 channels -> 32 (zero-padded channels change LayerNorm statistics,
    # so the padding carries the mean and spread of the two real ones: the
    # two-channel vectors [-1, 1] / [1, -1] become 16 copies of each value)
    f = torch.tensor(g["features"], dtype=torch.float32)                 # [1,2,2,2]
    feat = f.repeat_interleave(16, dim=-1)                               # [1,2,2,32]
    bfeat = torch.tensor(g["bias_features"], dtype=torch.float32).repeat_interleave(2, dim=-1)
    C, CB = 32, 4
    w = torch.zeros(C, 32)
    w[:16, 0] = -1.0 / 16
    w[16:, 0] = 1.0 / 16            # -mean of first half + mean of second half = (-x0 + x1) of the example
    par = {"norm_scale": torch.ones(C), "norm_bias": torch.zeros(C),
           "bias_norm_scale": torch.ones(CB), "bias_norm_bias": torch.zeros(CB),
           # the head is 32 wide here (logits scaled by 1/sqrt(2*32) instead of
           # 1/sqrt(2)): q and k carry a factor 32**0.25 each, v none
           "w_q": w * 32 ** 0.25, "w_k": w * 32 ** 0.25, "w_v": w.clone(),
           "w_bias": torch.zeros(CB, 1),
           "w_gate": torch.zeros(C, 32), "w_out": torch.zeros(32, C), "b_out": torch.zeros(C)}
    par["w_out"][0, 0], par["w_out"][0, 1] = 2.0, 4.0
    par["b_out"][0], par["b_out"][1] = 1.0, -1.0
    cu = lambda d: {k: v.cuda().contiguous() for k, v in d.items()}
    out = tied_row_attention(cu({"features": feat, "bias_features": bfeat}), cu(par),
                             eps=g["eps"])
    torch.cuda.synchronize()
    got = out[0, :, :, :2].double().cpu().numpy()
    exp = np.array([[[2, 1], [2, 1]], [[2 - 2 * p_, 1 - 4 * p_], [2 * p_, 4 * p_ - 3]]])
    np.testing.assert_allclose(got, exp, rtol=1e-5, atol=1e-5)


def test_tied_row_attention_full_size():
    """The benchmarked size (B=1, L=256, C=128, CB=128, H=4, D=32, bf16)."""
    from windowed_atom_attention_amd import tied_row_attention
    from windowed_atom_attention_amd.workloads import make_tied_workload
    acts, par = make_tied_workload()
    cu = lambda d: {k: v.cuda() for k, v in d.items()}
    got = tied_row_attention(cu(acts), cu(par))
    torch.cuda.synchronize()
    _tied_check(acts, par, got, RTOL[torch.bfloat16])


def test_mixed_local_and_scattered_key_tables():
    """One call whose first atoms use local windows (slot kernel) and whose
    later atoms select keys anywhere in the batch (gather kernel)."""
    w = make_workload("1", A=3000)
    ki = w.structure["key_index"].clone()
    g = torch.Generator().manual_seed(3)
    ki[:, 1504:] = torch.randint(-1, 3000, ki[:, 1504:].shape, generator=g)
    w.structure["key_index"] = ki
    gpu = run_gpu(w)
    ref = oracle.block(**w.kwargs(), intermediates=True)
    exact_zero_checks(w, gpu, ref["usable"], ref["allowed"])
    compare_block(w, gpu, ref)


@pytest.mark.parametrize("style", ["af3", "esmfold2"])
def test_slot_attention_step_scattered_keys(style):
    w = make_workload("4a" if style == "af3" else "4b", A=2000, dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(8)
    ki = torch.randint(-2, 2002, w.structure["key_index"].shape, generator=g)
    ki[:, :, 1] = ki[:, :, 0]
    ref_masks = oracle.block(**w.kwargs(), intermediates=True)
    B, A, H = w.dims["B"], w.dims["A"], w.dims["H"]
    HD = H * w.dims["D"]
    q, k, v = (torch.randn((B, A, HD), generator=g).to(torch.bfloat16) for _ in range(3))
    usable = torch.from_numpy(ref_masks["usable"]).bool()
    pair = pair_scale = w_pair = None
    if style == "af3":
        # the recipe's NaN rows sit on its own missing slots; with the new
        # ids some of those slots are allowed, so give every row a value
        pair = torch.nan_to_num(w.activations["pair"], nan=0.5)
        pair_scale, w_pair = w.parameters["pair_scale"], w.parameters["w_pair"]
    kw = dict(eps=w.eps, style=style, radius=-1)
    ref = oracle.slot_attention(q, k, v, usable, ki, w.masks["window_mask"], heads=H,
                                pair=pair, pair_scale=pair_scale, w_pair=w_pair, **kw)
    cu = lambda t: None if t is None else t.cuda()
    att, o = gpu_slot_attention(cu(q), cu(k), cu(v), cu(usable), cu(ki),
                                cu(w.masks["window_mask"]), heads=H, pair=cu(pair),
                                pair_scale=cu(pair_scale), w_pair=cu(w_pair), **kw)
    rtol = RTOL[torch.bfloat16]
    al = ref["allowed"].astype(bool)
    attn = np64(att)
    assert np.all(attn[np.broadcast_to(~al[:, None], attn.shape)] == 0.0)
    assert_close_rel("attention", attn, ref["attention"], rtol)
    assert_close("o", np64(o), ref["o"], rtol)
