"""Reader for the hand-worked block fixtures in tests/golden/."""
import glob
import os
import re

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _value(tok: str) -> float:
    m = re.fullmatch(r"(-?[0-9.]+)\*2\^(-?[0-9]+)", tok)
    if m:
        return float(m.group(1)) * 2.0 ** int(m.group(2))
    return float(tok)


def load(path: str) -> dict:
    out = {"name": os.path.basename(path)}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(":")
            toks = rest.split()
            if key == "format":
                out["format"] = toks[0]
            elif key in ("weights", "dequant"):
                vals = [_value(t) for t in toks]
                arr = np.array(vals, dtype=np.float64)
                if key == "weights":
                    w32 = arr.astype(np.float32)
                    assert np.array_equal(w32.astype(np.float64), arr), f"{path}: weight not exact in fp32"
                    arr = w32
                out[key] = arr
            elif key == "bytes":
                out["bytes"] = np.array([int(t, 16) for t in toks], dtype=np.uint8)
    return out


def all_blocks():
    return [load(p) for p in sorted(glob.glob(os.path.join(GOLDEN, "*.txt"))) if not p.endswith("README.txt")]


def load_shortlist(path: str) -> dict:
    """A hand-worked bound-copy row (tests/golden/shortlist/): K, the Q8_0
    block scales and quants of one row (blocks not listed are all zero), the
    residual norm E and the expected bytes."""
    out = {"name": os.path.basename(path), "q": {}}
    raw = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(":")
            toks = rest.split()
            if key == "k":
                out["k"] = int(toks[0])
            elif key == "d":
                out["d"] = np.array([_value(t) for t in toks], dtype=np.float64)
            elif key == "E":
                out["E"] = _value(toks[0])
            elif key == "bytes":
                raw += [int(t, 16) for t in toks]
            elif re.fullmatch(r"q[0-9]+", key):
                out["q"][int(key[1:])] = [int(t) for t in toks]
    nb = out["k"] // 32
    d = out["d"].astype(np.float16)
    assert np.array_equal(d.astype(np.float64), out["d"]), f"{path}: scale not exact in fp16"
    q = np.zeros((1, nb, 32), np.int8)
    for b, vals in out["q"].items():
        q[0, b] = vals
    out["fields"] = {"d": d[None, :], "q": q}
    out["bytes"] = np.array(raw, dtype=np.uint8)
    return out


def all_shortlist_rows():
    return [load_shortlist(p) for p in sorted(glob.glob(os.path.join(GOLDEN, "shortlist", "*.txt")))]
