"""Readers for the hand-derived fixture files in this folder (citations are in
each file's header)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _lines(name):
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [p.strip() for p in line.split("|")]


def _codes(text):
    out = []
    for part in text.split(","):
        part = part.strip()
        if "x" in part:
            n, c = part.split("x")
            out += [int(c)] * int(n)
        else:
            out.append(int(part))
    return out


def byte_vectors(name):
    """[(codes list, bytes)] from int3_byte_vectors.txt / int4_byte_vectors.txt."""
    return [(_codes(c), bytes.fromhex(b)) for c, b in _lines(name)]


def gemv_closed_forms():
    return {name: (int(K), float(y)) for name, K, y in _lines("gemv_closed_forms.txt")}


def tiny_moe():
    return {k: v for k, v in _lines("tiny_moe.txt")}


def _values(text):
    out = []
    for part in text.split(","):
        part = part.strip()
        if "x" in part:
            n, v = part.split("x")
            out += [float(v)] * int(n)
        else:
            out.append(float(part))
    return out


def rtn_int3(name="rtn_int3.txt"):
    """[(name, weights, scale bits, status, bytes)] from rtn_int3.txt (fp16
    scales) or rtn_int3_bf16.txt (bfloat16 scales)."""
    return [(n, _values(w), int(s, 16), int(st), bytes.fromhex(b))
            for n, w, s, st, b in _lines(name)]
