"""Readers for the hand-worked fixtures under tests/golden/."""
import os

import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.strip()
            if line and not line.startswith("#"):
                yield line


def row_tensor(dtype: str, patterns):
    """A one-row logits tensor holding exact bit patterns (hex strings)."""
    if dtype == "f32":
        v = torch.tensor([int(p, 16) for p in patterns], dtype=torch.int64).to(torch.int32)
        return v.view(torch.float32).reshape(1, -1).clone()
    v = torch.tensor([int(p, 16) for p in patterns], dtype=torch.int64).to(torch.int16)
    return v.view(torch.bfloat16).reshape(1, -1).clone()


def argmax_cases():
    """[(name, dtype, vocab, row tensor, expected id, expected value bits)]"""
    out = []
    for i, line in enumerate(_lines("argmax_cases.txt")):
        head, elems, want = [p.strip() for p in line.split("|")]
        dt, v = head.split()
        wid, wbits = want.split()
        out.append((f"case{i}", dt, int(v), row_tensor(dt, elems.split()), int(wid), int(wbits, 16)))
    return out


def block_stats_cases():
    """[(V, W, S, B, M, fp32 row tensor, [(bits, id) in rank order], combined id)]"""
    out = []
    for line in _lines("block_stats_cases.txt"):
        head, vals, stats, comb = [p.strip() for p in line.split("|")]
        v, w, s, b, m = (int(t) for t in head.split())
        row = torch.tensor([float(t) for t in vals.split()], dtype=torch.float32).reshape(1, -1)
        st = []
        for t in stats.split():
            bits, sid = t.split(":")
            st.append((int(bits, 16), int(sid)))
        out.append((v, w, s, b, m, row, st, int(comb)))
    return out


def verify_cases():
    """[(K, targets, drafts, out_tokens, sampled, rejected)]"""
    out = []
    for line in _lines("verify_cases.txt"):
        k, tg, dr, ot, cnt = [p.strip() for p in line.split("|")]
        ns, nr = (int(t) for t in cnt.split())
        out.append((int(k), [int(t) for t in tg.split()], [int(t) for t in dr.split()],
                    [int(t) for t in ot.split()], ns, nr))
    return out


def epilogue_cases():
    """([(value bits, scale float, expected bits)], [(d2t list, ids, expected)])"""
    import struct
    scales, maps = [], []
    for line in _lines("epilogue_cases.txt"):
        kind, a, b, c = [p.strip() for p in line.split("|")]
        if kind == "scale":
            scale = struct.unpack("<f", struct.pack("<I", int(b, 16)))[0]
            scales.append((int(a, 16), scale, int(c, 16)))
        else:
            maps.append(([int(t) for t in a.split()], [int(t) for t in b.split()],
                         [int(t) for t in c.split()]))
    return scales, maps


def ragged_verify_cases():
    """[(cu, targets, drafts, out_tokens, sampled, rejected, prefilling)] as int
    lists; prefilling is None where a case gives no flags."""
    out = []
    for line in _lines("ragged_verify_cases.txt"):
        fields = [[int(t) for t in p.split()] for p in line.split("|")]
        if len(fields) == 6:
            fields.append(None)
        assert len(fields) == 7, line
        out.append(tuple(fields))
    return out


def synthetic_verify_cases():
    """[(cu, targets, drafts, accept, out_tokens, sampled, rejected, prefilling)]
    as int lists; prefilling is None where a case gives no flags."""
    out = []
    for line in _lines("synthetic_verify_cases.txt"):
        fields = [[int(t) for t in p.split()] for p in line.split("|")]
        if len(fields) == 7:
            fields.append(None)
        assert len(fields) == 8, line
        out.append(tuple(fields))
    return out
