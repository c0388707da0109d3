"""Reader for the hand-worked text fixtures under tests/golden/."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bf16_exact_bits(v: float) -> int:
    """bf16 bit pattern of v, which must be exactly representable."""
    f = np.array([v], np.float32)
    u = int(f.view(np.uint32)[0])
    exact = float(f[0]) == v or (np.isinf(v) and np.isinf(f[0]))
    if (u & 0xFFFF) != 0 or not exact:
        raise ValueError(f"{v!r} is not exactly a bf16 value")
    return u >> 16


def _number(tok: str) -> float:
    """A decimal, or a C99 hexadecimal float such as 0x1p-121 or -0xffp-130."""
    return float.fromhex(tok) if "0x" in tok.lower() else float(tok)


def read_cases(name: str, width: int = 32):
    """Parse a fixture: list of dicts with 'name', 'bits' (uint16[width]) and fields."""
    cases = []
    cur = None
    with open(os.path.join(GOLDEN, name)) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            rest = rest.strip()
            if key == "case":
                cur = {"name": rest.split()[0]}
                cases.append(cur)
            elif key == "values":
                vals = []
                fill = 0.0
                for tok in rest.split():
                    if tok.startswith("rest="):
                        fill = _number(tok[5:])
                    else:
                        vals.append(_number(tok))
                vals += [fill] * (width - len(vals))
                assert len(vals) == width, (cur, len(vals))
                cur["values"] = vals
                cur["bits"] = np.array([_bf16_exact_bits(v) for v in vals], np.uint16)
            elif key == "codes":
                cur["codes"] = np.array([int(t) for t in rest.split()], np.int64)
                assert cur["codes"].size == width
            elif key in ("scale", "sx"):
                cur[key] = int(rest, 16)
            else:
                cur[key] = int(rest, 0)
    return cases
