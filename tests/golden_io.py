"""Readers for the hand-derived fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok: str) -> float:
    tok = tok.strip()
    if "0x" in tok.lower():
        return float.fromhex(tok)
    return float(tok)


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def e4m3_encode_cases():
    out = []
    for line in _lines("e4m3_encode.txt"):
        parts = line.split()
        out.append((_num(parts[0]), int(parts[1], 16), " ".join(parts[2:])))
    return out


def quantize_cases():
    cases, cur = [], {}
    for line in _lines("quantize_rows.txt"):
        key, val = line.split(":", 1)
        if key == "x":
            cur = {"x": [_num(t) for t in val.split()]}
        elif key == "scale":
            cur["scale"] = _num(val)
        elif key == "codes":
            cur["codes"] = [int(t, 16) for t in val.split()]
            cases.append(cur)
    return cases


def attention_case():
    rec = {"out": {}}
    for line in _lines("attention_tiny.txt"):
        key, val = line.split(":", 1)
        if key in ("k", "v"):
            rec[key] = [[_num(t) for t in row.split()] for row in val.split(";")]
        elif key == "q":
            rec["q"] = [_num(t) for t in val.split()]
        elif key == "sm_scale":
            rec["sm_scale"] = _num(val)
        else:
            rec["out"][key] = [_num(t) for t in val.split()]
    return rec
