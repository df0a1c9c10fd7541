"""Reader for the hand-derived fixtures in tests/golden/."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _parse_inputs(spec: str) -> np.ndarray:
    spec = spec.strip()
    if spec.startswith("@"):
        head, *items = spec.split()
        n = int(head[1:])
        out = np.zeros(n, dtype=np.float64)
        for it in items:
            k, v = it.split("=")
            if k == "all":
                out[:] = float.fromhex(v)
            else:
                out[int(k)] = float.fromhex(v)
    else:
        out = np.array([float.fromhex(v) for v in spec.split(",")], dtype=np.float64)
    h = out.astype(np.float16)
    assert np.array_equal(h.astype(np.float64), out) or np.isnan(out).any(), \
        "golden inputs must be exact binary16 values"
    return h


def tree_examples():
    """[(name, x_f16, tree, sequential, exact_f32, note)] from the worked-example file."""
    rows = []
    with open(os.path.join(GOLDEN, "fixed_tree_worked_examples.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, inputs, tree, seq, exact, note = [p.strip() for p in line.split("|", 5)]
            rows.append((name, _parse_inputs(inputs), np.float32(float.fromhex(tree)),
                         np.float32(float.fromhex(seq)), np.float32(float.fromhex(exact)), note))
    return rows


def bits32(v) -> int:
    return int(np.asarray(v, dtype=np.float32).view(np.uint32))
