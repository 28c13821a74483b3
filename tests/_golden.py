"""Parser for the hand-worked fixtures under tests/golden/ (no arithmetic of the method)."""
from __future__ import annotations

import os
import struct
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expand(tokens):
    out = []
    for t in tokens:
        # "v*n" repeats v n times, unless it is a product "A*2^B"
        if "*" in t and "^" not in t.split("*")[-1]:
            v, n = t.rsplit("*", 1)
            out.extend([v] * int(n))
        else:
            out.append(t)
    return out


def parse_value(tok: str):
    """Exact value of a token: Fraction, or the strings 'inf', '-inf', 'nan', '-0',
    or ('bits', int) for a 0x pattern."""
    t = tok.strip()
    if t.lower().startswith("0x"):
        return ("bits", int(t, 16))
    if t in ("inf", "-inf", "nan", "-0"):
        return t
    neg = t.startswith("-")
    if neg:
        t = t[1:]
    if "*2^" in t:
        a, b = t.split("*2^")
        v = Fraction(a) * Fraction(2) ** int(b)
    elif t.startswith("2^"):
        v = Fraction(2) ** int(t[2:])
    else:
        v = Fraction(t)
    return -v if neg else v


def bf16_bits_of_exact(v) -> int:
    """bf16 bit pattern of an exactly representable value token (no rounding allowed)."""
    if isinstance(v, tuple):
        return v[1]
    if v == "inf":
        return 0x7F80
    if v == "-inf":
        return 0xFF80
    if v == "nan":
        return 0x7FC0
    if v == "-0":
        return 0x8000
    f = float(v)
    if Fraction(f) != v:
        raise ValueError(f"{v} is not exact in binary64")
    w = struct.unpack("<I", struct.pack("<f", f))[0]
    if Fraction(struct.unpack("<f", struct.pack("<I", w))[0]) != v or (w & 0xFFFF):
        raise ValueError(f"{v} is not exact in bf16")
    return w >> 16


def f32_bits_of_exact(v) -> int:
    if isinstance(v, tuple):
        return v[1]
    f = float(v)
    w = struct.unpack("<I", struct.pack("<f", f))[0]
    if Fraction(struct.unpack("<f", struct.pack("<I", w))[0]) != v:
        raise ValueError(f"{v} is not exact in binary32")
    return w


def _fields(line):
    parts = [p.strip() for p in line.split("|")]
    head = parts[0].split()
    fields = {}
    for p in parts[1:]:
        k, v = p.split(":", 1)
        fields[k.strip()] = v.strip()
    return head[0], head[1], fields


def load_mx_cases(name="mx_worked_blocks.txt"):
    blocks, decodes = [], []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, name, fl = _fields(line)
            if kind == "block":
                x = [bf16_bits_of_exact(parse_value(t)) for t in _expand(fl["x"].split())]
                q = [int(t, 16) for t in _expand(fl["q"].split())]
                y = [bf16_bits_of_exact(parse_value(t)) for t in _expand(fl["y"].split())]
                assert len(x) == len(q) == len(y) == 32, name
                blocks.append(dict(name=name, x=x, s=int(fl["s"], 16), q=q, y=y))
            elif kind == "decode":
                decodes.append(dict(name=name, q=int(fl["q"], 16), s=int(fl["s"], 16), y=int(fl["y"], 16)))
            else:
                raise ValueError(kind)
    return blocks, decodes


def load_group_cases():
    cases = []
    with open(os.path.join(GOLDEN, "group_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, name, fl = _fields(line)
            assert kind == "group"
            M, K = int(fl["M"]), int(fl["K"])
            ends = [int(t) for t in fl["ends"].split()]
            rows = [r.split() for r in fl["x"].split(";")]
            x = [[bf16_bits_of_exact(parse_value(t)) for t in r] for r in rows]
            srows = [r.split() for r in fl["scales"].split(";")]
            scales = [[f32_bits_of_exact(parse_value(t)) for t in r] for r in srows]
            q = [[int(t, 16) for t in r.split()] for r in fl["q"].split(";")]
            assert len(x) == M and all(len(r) == K for r in x), name
            assert len(scales) == len(ends) and len(q) == M, name
            cases.append(dict(name=name, M=M, K=K, ends=ends, x=x, scales=scales, q=q))
    return cases
