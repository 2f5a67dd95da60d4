"""A CPU model of the statistics kernels' index arithmetic
(vocab_argmax_amd/csrc/block_stats.hip, and chunk_stats.hip further down),
checked over random geometries:

- the item decode covers every (row, shard, slot) of a launch exactly once
  and every statistic index lies inside [0, n_local * n_rows * M);
- within a segment, the edge elements read one by one and the 16-byte
  vectors of the pipelined scan (clamped chunk indices) touch only the
  segment's valid columns of its row, and cover them exactly;
- every vector address is 16-byte aligned, whatever the buffer's offset;
- the positions the fold packs decode back to the column that was loaded.

The model restates the kernel's integer formulas; it shares no code with
the library (none could be shared: the kernel is device code).  A change to
the kernel's indexing has to be carried over here.
"""
import random

import pytest

LANE_ITERS = 16            # VPA_LANE_ITERS
PIPE = {2: 8, 4: 16}       # VPA_PIPE_BF16, VPA_PIPE_F32


def slots(w, s, b):
    return max((i * w + w - 1) // b - (i * w) // b + 1 for i in range(s))


def lanes_log2(block, shard_width, esize):
    span = min(block, shard_width)
    vectors = (span * esize + 15) // 16 + 1
    lg = 3
    while lg < 6 and (1 << (lg + 1)) * LANE_ITERS <= vectors:
        lg += 1
    return lg


def decode_item(item, m, n_local):
    j = item % m
    rest = item // m
    return rest // n_local, rest % n_local, j          # (i, sl, j)


def segment_range(first_shard, sl, j, w, block, vocab):
    shard_lo = (first_shard + sl) * w
    blo = (shard_lo // block + j) * block
    lo = max(blo, shard_lo)
    hi = min(blo + block, shard_lo + w, vocab)
    return lo, hi


def scan_segment(esize, base_mod16, row, ld, col0, lo, hi, lanes):
    """Columns the group of `lanes` lanes reads for segment [lo, hi), with
    checks on every index; returns the multiset of columns as a list."""
    vec = 16 // esize
    mis = base_mod16 // esize
    a_lo = row * ld + (lo - col0) + mis
    d = lo - a_lo
    qa = -(-a_lo // vec)
    qb = (a_lo + (hi - lo)) // vec
    if qa < qb:
        head_end, tail_lo = qa * vec + d, qb * vec + d
    else:
        head_end, tail_lo, qb = hi, hi, qa
    cols = []
    for gl in range(lanes):                       # edge elements, one by one
        c = lo + gl
        while c < head_end:
            cols.append(c)
            c += lanes
        c = tail_lo + gl
        while c < hi:
            cols.append(c)
            c += lanes
    n = qb - qa
    if n > 0:
        u_deep = PIPE[esize]
        nit = -(-n // lanes)
        chunks = -(-nit // u_deep)
        c0 = qa * vec + d
        seen = set()
        for gl in range(lanes):
            for ch in range(chunks):
                i0 = gl + lanes * u_deep * ch
                for u in range(u_deep):
                    i = min(i0 + lanes * u, n - 1)           # load_clamped
                    assert 0 <= i < n
                    # byte address modulo 16: the kernel steps back `mis`
                    # elements from the buffer base, then adds whole vectors
                    addr = base_mod16 - mis * esize + (qa + i) * 16
                    assert addr % 16 == 0
                    # fold: the packed position decodes to the loaded vector
                    for e in range(vec):
                        pos = u * vec + e
                        i_dec = min(i0 + lanes * (pos // vec), n - 1)
                        assert i_dec == i
                        col = c0 + i_dec * vec + pos % vec
                        assert col == (qa + i) * vec + e + d
                    seen.add(i)
        for i in seen:
            cols.extend((qa + i) * vec + e + d for e in range(vec))
    # the buffer element of each column lies inside its row's valid part
    for c in cols:
        assert lo <= c < hi, (lo, hi, c)
        elem = row * ld + (c - col0)
        assert row * ld <= elem < row * ld + ld
    return cols


def check_launch(rng, esize):
    s = rng.choice([1, 2, 3, 4, 5, 8])
    vocab = rng.choice([1, 2, 7, 63, 1000, 4097, 50257, 70001, 151936, 200064])
    w = -(-vocab // s) + rng.choice([0, 0, 1, 3, 64])
    block = rng.choice([1, 3, 64, 255, 256, 1000, 1024, 2048, 4096, 8192, 65536, 1 << 20])
    if vocab > 5000 and block < 256:
        block = 256
    first = rng.randrange(s)
    n_local = rng.randint(1, s - first)
    col0 = first * w
    need = min(n_local * w, vocab - col0)
    ld = max(need, 1) + rng.choice([0, 0, 1, 5, 8, 128])
    base_mod16 = rng.choice([0, esize, 2 * esize, 16 - esize, 6 if esize == 2 else 12])
    m = slots(w, s, block)
    n_rows = rng.choice([1, 2, 3])
    lg = lanes_log2(block, w, esize)
    lanes = 1 << lg
    per_wave = 64 // lanes
    n_items = n_rows * n_local * m
    n_waves = -(-n_items // per_wave)
    seen_items, stat_idx = set(), set()
    segments = 0
    for wave in range(n_waves):
        for g in range(per_wave):
            item = wave * per_wave + g
            if item >= n_items:
                continue
            seen_items.add(item)
            i, sl, j = decode_item(item, m, n_local)
            idx = (sl * n_rows + i) * m + j
            assert 0 <= idx < n_local * n_rows * m
            stat_idx.add(idx)
            lo, hi = segment_range(first, sl, j, w, block, vocab)
            if lo >= hi:
                continue
            row = i
            cols = scan_segment(esize, base_mod16, row, ld, col0, lo, hi, lanes)
            assert sorted(cols) == list(range(lo, hi))     # each column exactly once
            segments += 1
    assert seen_items == set(range(n_items))
    assert len(stat_idx) == n_items
    return segments


@pytest.mark.parametrize("esize", [2, 4])
def test_statistics_kernel_index_arithmetic(esize):
    rng = random.Random(1000 + esize)
    segments = 0
    for _ in range(80):
        segments += check_launch(rng, esize)
    assert segments > 1000


def _source(name):
    import os
    return open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                             "vocab_argmax_amd", "csrc", name)).read()


def test_model_matches_the_kernel_constants():
    """The constants the model assumes are the ones the kernel source sets."""
    src = _source("block_stats.hip")
    assert "#define VPA_LANE_ITERS 16" in src
    assert "#define VPA_PIPE_BF16 8" in src
    assert "#define VPA_PIPE_F32 16" in src
    assert "i = i < ilast ? i : ilast;" in _source("vpa_scan.h")   # clamped chunk indices


# The chunked statistics of vpa_top_tokens (chunk_stats.hip) for bf16
# batches of up to CHUNK_MAX_BYTES: chunk c of the flattened (row, chunk)
# space is columns [q*CHUNK_COLS, min((q+1)*CHUNK_COLS, V)) of row c // Q,
# Q = ceil(V / CHUNK_COLS), read by wavefront c mod W; its statistic goes to
# stats[c].  The host takes this path only for V and ld multiples of 8 and a
# 16-byte aligned base (api.hip, chunk_sizes).
CHUNK_LOADS = 8                         # kChunkLoads
CHUNK_COLS = 64 * 8 * CHUNK_LOADS       # kChunkCols
CHUNK_MAX_BYTES = 1024 * 200064 * 2     # kChunkMaxBytes
GROUPS_PER_CU = 2                       # kGroupsPerCU


def chunk_sizes(vocab, ld, n_rows):
    return vocab % 8 == 0 and ld % 8 == 0 and 0 < n_rows <= CHUNK_MAX_BYTES // (2 * vocab)


def check_chunk_launch(rng):
    vocab = 8 * rng.choice([1, 2, 3, rng.randint(1, 600), rng.randint(500, 40000), 25008])
    ld = vocab + 8 * rng.choice([0, 0, 1, rng.randint(0, 300)])
    n_rows = rng.randint(1, min(CHUNK_MAX_BYTES // (2 * vocab), 40))
    assert chunk_sizes(vocab, ld, n_rows)
    per_row = -(-vocab // CHUNK_COLS)
    n_chunks = n_rows * per_row
    cus = rng.choice([1, 3, 80, 256, 304])
    groups = min(GROUPS_PER_CU * cus, -(-n_chunks // 4))
    n_waves = groups * 4
    visited = [0] * n_chunks
    spans = {}                                            # row -> [(lo, hi)]
    for wave in range(n_waves):
        for c in range(wave, n_chunks, n_waves):
            visited[c] += 1
            row = c // per_row
            col0 = (c - row * per_row) * CHUNK_COLS
            cols = min(vocab - col0, CHUNK_COLS)
            nv = cols // 8
            assert 0 <= row < n_rows and cols > 0 and cols % 8 == 0 and nv >= 1
            assert col0 % 8 == 0 and (row * ld + col0) % 8 == 0       # 16-byte aligned vectors
            # the loads: lane l, vector u reads vector min(l + 64u, nv - 1)
            last = max(min(lane + 64 * u, nv - 1) for lane in (0, 63) for u in (0, CHUNK_LOADS - 1))
            assert last == min(63 + 64 * (CHUNK_LOADS - 1), nv - 1)
            assert row * ld + col0 + last * 8 + 7 < row * ld + vocab   # valid columns only
            # fold decode of the last element a lane can pack (u = 7, e = 7)
            for lane in (0, 17, 63):
                pos = (CHUNK_LOADS - 1) * 8 + 7
                i = min(lane + 64 * (pos >> 3), nv - 1)
                assert col0 + i * 8 + (pos & 7) < vocab
            spans.setdefault(row, []).append((col0, col0 + nv * 8))
    assert visited == [1] * n_chunks                      # every statistic written once
    for row in range(n_rows):                             # the chunks tile [0, V) exactly
        got = sorted(spans[row])
        assert got[0][0] == 0 and got[-1][1] == vocab
        assert all(a[1] == b[0] for a, b in zip(got, got[1:]))
    return n_chunks


def test_chunk_statistics_index_arithmetic():
    rng = random.Random(2002)
    chunks = sum(check_chunk_launch(rng) for _ in range(120))
    assert chunks > 2000


def test_chunk_statistics_counts_fit_int32():
    """The largest eligible batch of any vocabulary stays far below 2^31
    chunks (the kernel and the combine index them with int32)."""
    for vocab in [8 * k for k in (1, 2, 7, 100, 512, 513, 25008, 2 ** 21 - 1)]:
        n_rows = CHUNK_MAX_BYTES // (2 * vocab)
        assert n_rows * -(-vocab // CHUNK_COLS) < 2 ** 31 // 8


def test_chunk_model_matches_the_kernel_constants():
    src = _source("chunk_stats.hip")
    assert "constexpr int kChunkLoads = 8;" in src
    assert "constexpr int kChunkCols = 64 * 8 * kChunkLoads;" in src
    assert "constexpr int kGroupsPerCU = 2;" in src
    assert "k.row = c / per_row;" in src and "k.col0 = (c - k.row * per_row) * kChunkCols;" in src
    assert "constexpr int64_t kChunkMaxBytes = (int64_t)1024 * 200064 * 2;" in _source("api.hip")
    assert "return v.vocab % 8 == 0 && ld % 8 == 0 && n_rows > 0 &&" in _source("api.hip")
