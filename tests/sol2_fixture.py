"""The hand-worked Sol-Attn2 fixture of tests/golden/sol2_groups.txt: its inputs and its
expected values (test infrastructure shared by the oracle pin and the kernel test)."""
import math
import os

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "sol2_groups.txt")
N = 96


def inputs(d: int = 4):
    """q, k, v [96, d] float64 holding the fixture's (bf16-exact) values; dims >= 4 are zero."""
    q = np.zeros((N, d))
    k = np.zeros((N, d))
    v = np.zeros((N, d))
    q[0:32, :4] = (3.5, 0, 1, 0)
    q[32:64, :4] = (3.5, 0, -1, 0)
    q[64:80, :4] = (-1, 3.5, 0, 0)
    q[80:96, :4] = (-1, 2.5, 0, 0)
    types = {"A": ((3.5, 0, 1, 0), (1, 0, 0, 0)), "B": ((0, 1, 0, 0), (0, 1, 0, 0)),
             "T": ((0.5, 1, -1, 0), (0, 0, 1, 0)), "U": ((0, 1.046875, 0, 0), (0, 0, 0, 1))}
    pattern = "ABBBBTTU"
    for u in range(64):
        kk, vv = types[pattern[u % 8]]
        k[u, :4] = kk
        v[u, :4] = vv
    k[64:96, :4] = (1.75, 1.75, 0, 0)
    v[64:96, :4] = (2, 2, 2, 2)
    return q, k, v


def load(d: int = 4) -> dict:
    """name -> float64 array of the expressions evaluated for head dimension d (s = 1/sqrt(d);
    ``mu1`` is bound to mu1_sink_a2)."""
    env = {"__builtins__": {}, "exp": math.exp, "log": math.log, "s": 1.0 / math.sqrt(d)}
    out = {}
    with open(PATH) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            name, expr = (s.strip() for s in line.split("=", 1))
            vals = np.array([float(eval(e, env)) for e in _split_top(expr)])
            out[name] = vals
            if name == "mu1_sink_a2":
                env["mu1"] = float(vals[0])
    return out


def _split_top(expr: str):
    """Split on the commas that are not inside parentheses."""
    parts, depth, cur = [], 0, ""
    for ch in expr:
        if ch == "(":
            depth += 1
        elif ch == ")":
            depth -= 1
        if ch == "," and depth == 0:
            parts.append(cur)
            cur = ""
        else:
            cur += ch
    parts.append(cur)
    return [p.strip() for p in parts if p.strip()]
