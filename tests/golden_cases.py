"""Loader for tests/golden/worked_cases.json (hand-built closed-form cases)."""

import json
import math
import os

import numpy as np
import torch

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_cases.json")
_ENV = {"exp": math.exp, "log": math.log, "log1p": math.log1p, "e": math.e, "sqrt": math.sqrt}


def _eval(expr):
    return float(eval(expr, {"__builtins__": {}}, _ENV))  # trusted, repo-local fixture


def _rows(spec, N, d):
    x = torch.zeros((N, d), dtype=torch.float32)
    for i, row in enumerate(spec):
        for j, val in row:
            x[i, j] = float(val)
    return x


def load():
    with open(_PATH) as f:
        doc = json.load(f)
    cases = []
    for c in doc["cases"]:
        N, d = c["N"], c["d"]
        q = _rows(c["q"], N, d)
        k = _rows(c["k"], N, d)
        v = torch.eye(N, d) if c.get("v_rows_onehot") else _rows(c["v"], N, d)
        to = lambda t: t.reshape(1, 1, N, d).to(torch.bfloat16)  # noqa: E731
        # every stored input is a small integer, so the bf16 rounding is exact
        assert torch.equal(to(q).float().reshape(N, d), q)
        o = np.zeros((N, d))
        for i, row in enumerate(c["o"]):
            for j, expr in enumerate(row):
                o[i, j] = _eval(expr)
        lse = np.array([_eval(e) for e in c["lse"]])
        cases.append(dict(name=c["name"], N=N, d=d, causal=c["causal"], scale=_eval(c["scale"]),
                          q=to(q), k=to(k), v=to(v), o=o, lse=lse))
    return cases
