"""Loader for the worked-example fixtures in tests/golden/.

Each fixture holds the example's inputs and the closed forms the page states
for its results, as small arithmetic expressions over named quantities."""
import json
import math
import os

import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_NS = {"exp": math.exp, "sqrt": math.sqrt, "pi": math.pi}


def _value(x, ns):
    if isinstance(x, list):
        return [_value(v, ns) for v in x]
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, ns))
    return x


def _tensor(spec, ns, dtype):
    if isinstance(spec, str):
        name, args = spec.split("(", 1)
        shape = [int(a) for a in args.rstrip(")").split(",")]
        if name == "zeros":
            return torch.zeros(shape, dtype=dtype)
        if name == "eye":
            return torch.eye(shape[0], dtype=dtype)
        raise ValueError(spec)
    return torch.tensor(_value(spec, ns), dtype=dtype)


def load(name, dtype=torch.float64):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    ns = dict(_NS)
    for k, v in g.get("define", {}).items():
        ns[k] = float(eval(v, {"__builtins__": {}}, ns))
    acts = {k: _tensor(v, ns, dtype) for k, v in g["activations"].items()}
    params = {k: _tensor(v, ns, dtype) for k, v in g["parameters"].items()}
    masks = {k: torch.tensor(v, dtype=torch.bool) for k, v in g["masks"].items()}
    structure = {k: torch.tensor(v, dtype=torch.int64) for k, v in g["structure"].items()}
    expected = {k: torch.tensor(_value(v, ns), dtype=torch.float64)
                for k, v in g["expected"].items()}
    return dict(fixture=g, ns=ns, activations=acts, parameters=params,
                masks=masks, structure=structure, expected=expected)
