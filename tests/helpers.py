"""Shared test helpers: golden-file parsing and comparison metrics.

Nothing here computes any part of the method; it only reads fixtures and
measures differences between two results.
"""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _ranges(text):
    text = text.strip()
    if not text or text == "none":
        return []
    out = []
    for part in text.split(","):
        a, b = part.split(":")
        out.append((int(a), int(b)))
    return out


def load_span_examples(path=None):
    """Parse spans_worked_examples.txt -> {name: {"T", "mask", "spans": {G: list},
    "bits": {BM: [words]}, "count": A}}."""
    path = path or os.path.join(GOLDEN, "spans_worked_examples.txt")
    cases = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, name, rest = (line.split(None, 2) + [""])[:3]
            if kind == "case":
                T_tok, act_tok = rest.split(None, 1) if " " in rest else (rest, "active=")
                T = int(T_tok.split("=")[1])
                mask = np.zeros(T, np.uint8)
                for a, b in _ranges(act_tok.split("=", 1)[1]):
                    mask[a:b] = 1
                cases[name] = {"T": T, "mask": mask, "spans": {}, "bits": {}, "count": None}
            elif kind == "spans":
                g_tok, sp = rest.split(None, 1)
                cases[name]["spans"][int(g_tok.split("=")[1])] = _ranges(sp)
            elif kind == "bits":
                bm_tok, words = rest.split(None, 1)
                cases[name]["bits"][int(bm_tok.split("=")[1])] = [int(w, 16) for w in words.split(",")]
            elif kind == "count":
                cases[name]["count"] = int(rest)
            else:
                raise ValueError(line)
    return cases


def rel_fro(got, ref):
    """||got - ref||_F / ||ref||_F (0/0 -> 0)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return float(num)
    return float(num / den)


def max_abs(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)))
