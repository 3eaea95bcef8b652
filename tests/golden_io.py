"""Readers for the hand-worked fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _matrix(spec: str) -> np.ndarray:
    rows = [r.split() for r in spec.split(";")]
    return np.array([[float(v) for v in r] for r in rows])


def linear_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "linear_tiny.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case "):
                cur = {"name": line.split()[1]}
                cases.append(cur)
                continue
            head, body = line.split(":", 1)
            name, shape = head.split()
            m = _matrix(body)
            assert m.shape == tuple(int(v) for v in shape.split("x")), line
            cur[name] = m
    return cases


def paging_case():
    d = {"tables": []}
    with open(os.path.join(GOLDEN, "paging_tiny.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key.startswith("table"):
                d["tables"].append(np.array([int(v) for v in vals], dtype=np.int32))
            elif key in ("block", "cap", "n_valid", "n_runs"):
                d[key] = int(vals[0])
            else:
                d[key] = np.array([int(v) for v in vals], dtype=np.int64)
    return d
