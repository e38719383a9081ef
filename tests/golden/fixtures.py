"""Parser for the hand-worked format examples in ``q1_format_examples.txt``."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _runs(tokens):
    out = []
    for t in tokens:
        c, v = t.split("x", 1)
        out.extend([float(v)] * int(c))
    return out


def load_cases(path=os.path.join(HERE, "q1_format_examples.txt")):
    cases, cur = [], None
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            if key == "case":
                cur = {"name": rest[0]}
                cases.append(cur)
            elif key == "K":
                cur["K"] = int(rest[0])
            elif key == "meta":
                cur["meta"] = rest[0]
            elif key == "words":
                cur["packed"] = np.array([[int(t, 16) for t in rest]], dtype=np.uint32)
            elif key == "scales":
                cur["scales"] = np.array([[int(t, 16) for t in rest]], dtype=np.uint16)
            elif key == "biases":
                cur["biases"] = None if rest == ["none"] else np.array([[int(t, 16) for t in rest]], dtype=np.uint16)
            elif key == "dequant":
                cur["dequant"] = np.array(_runs(rest), dtype=np.float64)
            elif key == "x":
                cur["x"] = np.array(_runs(rest), dtype=np.float64)
            elif key == "y":
                cur["y"] = float(rest[0])
            else:
                raise ValueError(f"unknown key {key}")
    return cases
