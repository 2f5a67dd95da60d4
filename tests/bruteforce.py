"""Pure-Python brute force for tiny inputs, formulated differently from the
oracle so that the two pin each other.

* argmax: the winner is the lowest column that no other valid column beats,
  found by comparing every pair (quadratic) -- the oracle instead keeps a
  running best in one left-to-right pass.
* block statistics: columns are grouped by (shard, global block) through a
  dictionary keyed on the column's own shard and block numbers; slot counts
  come from listing every column of the padded row -- the oracle instead walks
  slot ranges derived from the shard start.
* greedy verification: the accepted prefix is the longest run of equal
  (draft, target) pairs from the left (itertools.takewhile).
* synthetic acceptance: the emitted tokens are the list of accepted drafts
  with the next target appended, padded with -1 to K+1 entries; the counts
  are read off that list.

The rule itself (vLLM PR #62604, "Purpose" items 1 and 2): NaN beats every
number, ties go to the lowest id, -0 equals +0; blocks keep global
boundaries across shard edges.
"""
import itertools
import math
import struct

SENTINEL = (0xFF800000, 0x7FFFFFFF)


def f32_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]


def beats(a: float, b: float) -> bool:
    """a is strictly above b in the argmax order (NaN on top, -0 == +0)."""
    if math.isnan(a):
        return not math.isnan(b)
    if math.isnan(b):
        return False
    return a > b


def bf_argmax(bits):
    """Lowest column that no other column beats.  `bits` are fp32 patterns."""
    vals = [f32_value(b) for b in bits]
    for c, v in enumerate(vals):
        if not any(beats(w, v) for w in vals):
            return c, bits[c] & 0xFFFFFFFF
    raise AssertionError("some element is always maximal")


def bf_stats_slots(shard_width: int, n_shards: int, block: int) -> int:
    per_shard = {}
    for c in range(n_shards * shard_width):
        per_shard.setdefault(c // shard_width, set()).add(c // block)
    return max(len(v) for v in per_shard.values())


def bf_block_stats(bits, vocab, shard_width, n_shards, block):
    """Statistics of one padded row as {(shard, slot): (value_bits, id)} plus M."""
    m = bf_stats_slots(shard_width, n_shards, block)
    groups = {}
    for c in range(vocab):
        s = c // shard_width
        b = c // block
        groups.setdefault((s, b), []).append(c)
    out = {}
    for s in range(n_shards):
        first_block = (s * shard_width) // block
        for j in range(m):
            cols = groups.get((s, first_block + j), [])
            if cols:
                w, vb = bf_argmax([bits[c] for c in cols])
                out[(s, j)] = (vb, cols[w])
            else:
                out[(s, j)] = SENTINEL
    return out, m


def bf_verify(targets, drafts):
    """(out_tokens, sampled, rejected) for one request; targets has K+1 entries."""
    k = len(drafts)
    n = len(list(itertools.takewhile(lambda p: p[0] == p[1], zip(drafts, targets))))
    out = list(drafts[:n]) + [targets[n]] + [-1] * (k - n)
    return out, n + 1, k - n


def bf_verify_synthetic(targets, drafts, accept):
    """(out_tokens, sampled, rejected) for one request under an accept count:
    accept < 0 is the real greedy rule; otherwise the first accept drafts
    (at most K) are taken as they are, followed by the next target."""
    if accept < 0:
        return bf_verify(targets, drafts)
    k = len(drafts)
    taken = list(drafts[:accept])
    emitted = taken + [targets[len(taken)]]
    return emitted + [-1] * (k + 1 - len(emitted)), len(emitted), k - len(taken)
