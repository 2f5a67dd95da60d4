"""Pins of the oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with
  * the hand-worked fixtures in tests/golden/ (expected values worked out by
    hand from the rule of vLLM PR #62604, "Purpose" items 1 and 2);
  * the pure-Python brute force of tests/bruteforce.py, exhaustively over
    tiny rows drawn from an alphabet of special values;
  * torch.argmax on the CPU, the routine PR #62604 ("Purpose", item 2) names
    as the semantics of the fused get_top_tokens;
  * the invariant that the combined statistics give the full-row argmax for
    any shard count, shard width, block size and shard-edge placement, and
    that per-rank statistics concatenated in rank order equal the statistics
    of all shards at once (PR #62604, "Purpose" item 1 and "Test Plan");
  * the greedy acceptance rule, by brute force over every draft tuple of tiny
    vocabularies;
  * the epilogue of the combined argmax (draft-to-target map, positive scale)
    against hand-worked cases and torch's fp32 multiply;
  * synthetic acceptance (caller-given accept counts) against hand-worked
    cases, brute force over every draft tuple and count, and the invariants
    that a count equal to the real accepted length, or no count at all,
    changes nothing.
The same pins run against deliberately broken copies of the oracle
(tests/test_oracle_mutants.py) to show that each plausible mistake is caught.
"""
import itertools
import random

import torch

import bruteforce as bf
import golden_io

F32_ALPHABET = [0xFF800000, 0xBFC00000, 0x80000000, 0x00000000, 0x00000001, 0x00000002,
                0x3FC00000, 0x7F800000, 0x7FC00000, 0xFFC12300]
BF16_ALPHABET = [0xFF80, 0xBFC0, 0x8000, 0x0000, 0x0001, 0x0002, 0x3FC0, 0x7F80, 0x7FC0, 0xFFC1]


def bits_of(x: torch.Tensor):
    """fp32 bit patterns of every element (bf16 widened) as an int64 tensor."""
    if x.dtype == torch.float32:
        return x.contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    return (x.contiguous().view(torch.int16).to(torch.int64) & 0xFFFF) << 16


def rows_from_patterns(patterns, dtype):
    if dtype == torch.float32:
        t = torch.tensor(patterns, dtype=torch.int64).to(torch.int32)
        return t.view(torch.float32)
    t = torch.tensor(patterns, dtype=torch.int64).to(torch.int16)
    return t.view(torch.bfloat16)


def pin_golden_argmax(o):
    for name, dt, v, row, wid, wbits in golden_io.argmax_cases():
        ids, vals = o.argmax(row, v)
        assert (int(ids[0]), int(vals[0])) == (wid, wbits), (name, int(ids[0]), hex(int(vals[0])))


def pin_golden_block_stats(o):
    for v, w, s, b, m, row, want, comb in golden_io.block_stats_cases():
        assert o.stats_slots(w, s, b) == m, (v, w, s, b)
        st = o.block_stats(row, v, w, s, b)
        got = [(int(p[0]) & 0xFFFFFFFF, int(p[1])) for p in st.reshape(-1, 2)]
        assert got == want, (v, w, s, b, got)
        ids, _ = o.combine(st)
        assert int(ids[0]) == comb


def pin_golden_verify(o):
    for k, targets, drafts, out, ns, nr in golden_io.verify_cases():
        vocab = 16
        # full logits: row j has its only maximum at targets[j]
        x = torch.zeros((k + 1, vocab), dtype=torch.float32)
        for j, t in enumerate(targets):
            x[j, t] = 1.0
        d = torch.tensor([drafts], dtype=torch.int32)
        got = o.greedy_verify_logits(x, vocab, d)
        assert got[0][0].tolist() == out and int(got[1][0]) == ns and int(got[2][0]) == nr, \
            (k, targets, drafts, got)
        assert got[3][0].tolist() == targets
        # from statistics: one shard, one slot per row, holding the target
        dstat = torch.tensor([[[[0x3F800000, t]] for t in targets[:k]]], dtype=torch.int64)
        bstat = torch.tensor([[[[0x3F800000, targets[k]]]]], dtype=torch.int64)
        got = o.greedy_verify(dstat.to(torch.int32), bstat.to(torch.int32), d)
        assert got[0][0].tolist() == out and int(got[1][0]) == ns and int(got[2][0]) == nr


def pin_exhaustive_argmax(o):
    """Every row of length 1..4 over a 10-value alphabet of special values."""
    for dtype, alphabet in ((torch.float32, F32_ALPHABET), (torch.bfloat16, BF16_ALPHABET)):
        for length in range(1, 5):
            combos = list(itertools.product(alphabet, repeat=length))
            x = rows_from_patterns(combos, dtype)
            ids, vals = o.argmax(x, length)
            wide = bits_of(x).tolist()
            for r, row in enumerate(wide):
                want = bf.bf_argmax(row)
                got = (int(ids[r]), int(vals[r]))
                assert got == want, (dtype, [hex(b) for b in row], got, want)


def _special_matrix(n_rows, width, seed, dtype):
    """Rows mixing normal draws, heavy ties (values on a coarse grid), NaNs,
    infinities, signed zeros and all -inf rows."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((n_rows, width), generator=g)
    coarse = torch.randint(-3, 4, (n_rows, width), generator=g).float()
    pick = torch.rand((n_rows, width), generator=g)
    x = torch.where(torch.arange(n_rows)[:, None] % 3 == 1, coarse, x)
    x = torch.where(pick < 0.002, torch.full_like(x, float("nan")), x)
    x = torch.where((pick > 0.002) & (pick < 0.004), torch.full_like(x, float("inf")), x)
    x = torch.where((pick > 0.004) & (pick < 0.01), torch.full_like(x, float("-inf")), x)
    x = torch.where((pick > 0.01) & (pick < 0.02), torch.full_like(x, -0.0), x)
    if n_rows > 4:
        x[4] = float("-inf")
    return x.to(dtype)


def pin_torch_argmax(o):
    """ids equal torch.argmax over the valid columns (fp32 upcast); values are
    the bits of the chosen element."""
    for dtype in (torch.float32, torch.bfloat16):
        for seed, (n, width, vocab) in enumerate([(64, 333, 333), (32, 5000, 4990), (16, 70000, 69999)]):
            x = _special_matrix(n, width, 100 + seed, dtype)
            x[:, vocab:] = float("nan")
            ids, vals = o.argmax(x, vocab)
            want = torch.argmax(x[:, :vocab].float(), dim=1).to(torch.int32)
            assert torch.equal(ids, want), (dtype, n, width, (ids != want).nonzero()[:5])
            wb = bits_of(x).gather(1, want.long()[:, None])[:, 0]
            assert torch.equal(vals, wb)


def pin_slots(o):
    for w in range(1, 41):
        for s in range(1, 6):
            for b in (1, 2, 3, 4, 5, 7, 8, 16, 33, 64, 200):
                assert o.stats_slots(w, s, b) == bf.bf_stats_slots(w, s, b), (w, s, b)


def pin_block_stats_bruteforce(o):
    rng = random.Random(7)
    for trial in range(300):
        dtype = torch.float32 if trial % 2 == 0 else torch.bfloat16
        alphabet = F32_ALPHABET if dtype == torch.float32 else BF16_ALPHABET
        s = rng.randint(1, 5)
        w = rng.randint(1, 12)
        vocab = rng.randint(max(1, (s - 1) * w + 1), s * w)
        b = rng.randint(1, 2 * s * w + 1)
        pats = [rng.choice(alphabet) for _ in range(s * w)]
        x = rows_from_patterns([pats], dtype)
        st = o.block_stats(x, vocab, w, s, b)
        row_bits = bits_of(x)[0].tolist()
        want, m = bf.bf_block_stats(row_bits, vocab, w, s, b)
        assert st.shape[2] == m, (s, w, b, vocab, st.shape, m)
        for sh in range(s):
            for j in range(m):
                got = (int(st[sh, 0, j, 0]) & 0xFFFFFFFF, int(st[sh, 0, j, 1]))
                assert got == want[(sh, j)], (s, w, vocab, b, sh, j, got, want[(sh, j)])


def pin_invariance(o):
    """combine(block_stats) == full-row argmax for many geometries; rank-wise
    statistics concatenated in rank order == statistics of all shards."""
    rng = random.Random(11)
    for dtype in (torch.float32, torch.bfloat16):
        for vocab in (997, 5000):
            x_full = _special_matrix(12, vocab + 40, 500 + vocab, dtype)
            for _ in range(12):
                s = rng.randint(1, 9)
                w = -(-vocab // s) + rng.randint(0, 5)       # padded width S*W >= V
                b = rng.choice([1, 7, 64, 256, 1000, 1024, 4096, 8192, s * w, 10 * s * w])
                x = x_full[:, :s * w].contiguous()
                x[:, vocab:] = float("nan")
                want_ids, want_vals = o.argmax(x, vocab)
                st = o.block_stats(x, vocab, w, s, b)
                ids, vals = o.combine(st)
                assert torch.equal(ids, want_ids), (dtype, vocab, s, w, b)
                assert torch.equal(vals, want_vals)
                # each rank reduces only its own columns, with global ids
                parts = [o.block_stats(x[:, r * w:(r + 1) * w].contiguous(), vocab, w, s, b,
                                       first_shard=r, n_local=1) for r in range(s)]
                assert torch.equal(torch.cat(parts, 0), st), (dtype, vocab, s, w, b)
                # a row list picks rows out of order
                rows = torch.tensor([5, 0, 11, 5], dtype=torch.int32)
                st_rows = o.block_stats(x, vocab, w, s, b, rows=rows)
                assert torch.equal(st_rows, st[:, rows.long()])


def pin_verify_bruteforce(o):
    """Every draft tuple over {-1, 0..V-1}^K against every target tuple, V<=3, K<=3."""
    for vocab in (1, 2, 3):
        for k in (1, 2, 3):
            for targets in itertools.product(range(vocab), repeat=k + 1):
                x = torch.zeros((k + 1, vocab), dtype=torch.float32)
                for j, t in enumerate(targets):
                    x[j, t] = 1.0
                drafts = list(itertools.product(range(-1, vocab), repeat=k))
                n_req = len(drafts)
                xx = x.repeat(n_req, 1)
                d = torch.tensor(drafts, dtype=torch.int32)
                out, ns, nr, tg = o.greedy_verify_logits(xx, vocab, d)
                draft_rows, bonus_rows = _verify_rows(n_req, k)
                dst = o.block_stats(xx, vocab, vocab, 1, 1, rows=draft_rows)
                bst = o.block_stats(xx, vocab, vocab, 1, 1, rows=bonus_rows)
                out2, ns2, nr2, tg2 = o.greedy_verify(dst, bst, d)
                for r, dr in enumerate(drafts):
                    want = bf.bf_verify(list(targets), list(dr))
                    got = (out[r].tolist(), int(ns[r]), int(nr[r]))
                    got2 = (out2[r].tolist(), int(ns2[r]), int(nr2[r]))
                    assert got == want and got2 == want, (vocab, k, targets, dr, got, got2, want)
                    assert tg[r].tolist() == list(targets) == tg2[r].tolist()


def _verify_rows(n_req, k):
    r = torch.arange(n_req)[:, None] * (k + 1)
    draft = (r + torch.arange(k)[None, :]).reshape(-1).to(torch.int32)
    bonus = (torch.arange(n_req) * (k + 1) + k).to(torch.int32)
    return draft, bonus


def pin_golden_epilogue(o):
    scales, maps = golden_io.epilogue_cases()
    for bits, scale, want in scales:
        got = int(o.scale_bits(torch.tensor([bits]), scale)[0])
        assert got == want, (hex(bits), scale, hex(got), hex(want))
    for d2t, ids, want in maps:
        got = o.map_ids(torch.tensor(ids, dtype=torch.int32), torch.tensor(d2t)).tolist()
        assert got == want, (d2t, ids, got, want)


def pin_scale_matches_torch(o):
    """The scaled maximum equals torch's fp32 multiply on the CPU (IEEE, round
    to nearest, subnormals kept) for every non-NaN value."""
    g = torch.Generator().manual_seed(3)
    bits = torch.cat([torch.randint(0, 2**32, (3000,), generator=g, dtype=torch.int64),
                      torch.randint(0, 2**24, (1000,), generator=g, dtype=torch.int64),  # subnormals
                      torch.tensor([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF])])
    vals = bits.to(torch.int32).view(torch.float32)
    keep = ~torch.isnan(vals)
    for scale in (0.5, 0.7, 1.0, 1.4285714, 3.0, 1e-30, 7e30):
        s32 = torch.tensor(scale, dtype=torch.float32)
        want = (vals[keep] * s32).view(torch.int32).to(torch.int64) & 0xFFFFFFFF
        got = o.scale_bits(bits[keep], float(s32))
        assert torch.equal(got, want), scale


def _ragged_logits(targets, vocab):
    """Rows whose only maximum sits at the given target ids."""
    x = torch.zeros((len(targets), vocab), dtype=torch.float32)
    for i, t in enumerate(targets):
        x[i, t] = 1.0
    return x


def pin_ragged_verify(o):
    """Ragged verification: hand-worked cases (some with requests still
    prefilling); every request equals the brute-force greedy rule with its own
    K, or samples nothing when flagged as prefilling; flagging requests leaves
    every other request's outputs as they were; statistics and logits agree."""
    import oracle as _oracle
    for cu, targets, drafts, out, ns, nr, pf in golden_io.ragged_verify_cases():
        x = _ragged_logits(targets, 16)
        cu_t = torch.tensor(cu, dtype=torch.int32)
        d = torch.tensor(drafts, dtype=torch.int32)
        got = o.greedy_verify_ragged(x, 16, cu_t, d, prefilling=pf)
        assert got[0].tolist() == out and got[1].tolist() == ns and got[2].tolist() == nr, \
            (cu, pf, got)
        assert got[3].tolist() == targets
    rng = random.Random(5)
    for trial in range(200):
        vocab = rng.randint(1, 4)
        n_req = rng.randint(1, 6)
        ks = [rng.randint(0, 4) for _ in range(n_req)]
        cu = [0]
        for k in ks:
            cu.append(cu[-1] + k)
        targets = [rng.randrange(vocab) for _ in range(cu[-1] + n_req)]
        drafts = [rng.randint(-1, vocab - 1) for _ in range(cu[-1])]
        pf = [int(rng.random() < 0.3) for _ in range(n_req)] if trial % 2 else None
        x = _ragged_logits(targets, vocab)
        cu_t = torch.tensor(cu, dtype=torch.int32)
        d = torch.tensor(drafts, dtype=torch.int32)
        out, ns, nr, tg = o.greedy_verify_ragged(x, vocab, cu_t, d, prefilling=pf)
        draft_rows, bonus_rows = _oracle.ragged_rows(cu_t)
        dst = o.block_stats(x, vocab, vocab, 1, 1, rows=draft_rows)
        bst = o.block_stats(x, vocab, vocab, 1, 1, rows=bonus_rows)
        got2 = o.greedy_verify_ragged_stats(dst, bst, cu_t, d, prefilling=pf)
        for a, b in zip((out, ns, nr, tg), got2):
            assert torch.equal(a, b), (cu, drafts, pf)
        assert tg.tolist() == targets
        plain = o.greedy_verify_ragged(x, vocab, cu_t, d) if pf else None
        for r, k in enumerate(ks):
            base = cu[r] + r
            got = (out[base:base + k + 1].tolist(), int(ns[r]), int(nr[r]))
            if pf and pf[r]:
                assert got == ([-1] * (k + 1), 0, 0), (cu, r, got)
                continue
            want = bf.bf_verify(targets[base:base + k + 1], drafts[cu[r]:cu[r] + k])
            assert got == want, (cu, r, got, want)
            if plain is not None:
                # a flag on other requests changes nothing here
                assert got == (plain[0][base:base + k + 1].tolist(), int(plain[1][r]),
                               int(plain[2][r])), (cu, r, pf)


def _uniform_stats(o, x, vocab, n_req, k):
    """Draft and bonus statistics of a uniform batch (one shard, one-column blocks)."""
    draft_rows, bonus_rows = _verify_rows(n_req, k)
    return (o.block_stats(x, vocab, vocab, 1, 1, rows=draft_rows),
            o.block_stats(x, vocab, vocab, 1, 1, rows=bonus_rows))


def pin_synthetic_verify(o):
    """Synthetic acceptance: hand-worked cases through all four verification
    entry points; brute force over every target tuple, draft tuple in
    {-1..V-1}^K and count in {-2..K+1} (V <= 2, K <= 3); a count equal to the
    real accepted length reproduces the real outputs; counts that are all
    negative equal giving none; random ragged batches with counts and
    prefilling flags, request by request."""
    import oracle as _oracle
    for cu, targets, drafts, acc, out, ns, nr, pf in golden_io.synthetic_verify_cases():
        x = _ragged_logits(targets, 16)
        cu_t = torch.tensor(cu, dtype=torch.int32)
        d = torch.tensor(drafts, dtype=torch.int32)
        got = o.greedy_verify_ragged(x, 16, cu_t, d, prefilling=pf, accept=acc)
        assert (got[0].tolist(), got[1].tolist(), got[2].tolist()) == (out, ns, nr), \
            (cu, acc, pf, got)
        assert got[3].tolist() == targets
        draft_rows, bonus_rows = _oracle.ragged_rows(cu_t)
        dst = o.block_stats(x, 16, 16, 1, 1, rows=draft_rows)
        bst = o.block_stats(x, 16, 16, 1, 1, rows=bonus_rows)
        got2 = o.greedy_verify_ragged_stats(dst, bst, cu_t, d, prefilling=pf, accept=acc)
        for a, b in zip(got, got2):
            assert torch.equal(a, b), (cu, acc)
        ks = {cu[r + 1] - cu[r] for r in range(len(cu) - 1)}
        if pf is None and len(ks) == 1 and min(ks) > 0:
            k, n_req = ks.pop(), len(cu) - 1
            du = d.reshape(n_req, k)
            got3 = o.greedy_verify_logits(x, 16, du, accept=acc)
            got4 = o.greedy_verify(*_uniform_stats(o, x, 16, n_req, k), du, accept=acc)
            for g in (got3, got4):
                assert g[0].reshape(-1).tolist() == out and g[1].tolist() == ns \
                    and g[2].tolist() == nr, (cu, acc, g)
    for vocab in (1, 2):
        for k in (1, 2, 3):
            for targets in itertools.product(range(vocab), repeat=k + 1):
                x = torch.zeros((k + 1, vocab), dtype=torch.float32)
                for j, t in enumerate(targets):
                    x[j, t] = 1.0
                cases = [(dr, a) for dr in itertools.product(range(-1, vocab), repeat=k)
                         for a in range(-2, k + 2)]
                n_req = len(cases)
                xx = x.repeat(n_req, 1)
                d = torch.tensor([c[0] for c in cases], dtype=torch.int32)
                acc = [c[1] for c in cases]
                got = o.greedy_verify_logits(xx, vocab, d, accept=acc)
                got2 = o.greedy_verify(*_uniform_stats(o, xx, vocab, n_req, k), d, accept=acc)
                real = o.greedy_verify_logits(xx, vocab, d)
                same = o.greedy_verify_logits(xx, vocab, d, accept=real[1] - 1)
                for r, (dr, a) in enumerate(cases):
                    want = bf.bf_verify_synthetic(list(targets), list(dr), a)
                    for g in (got, got2):
                        assert (g[0][r].tolist(), int(g[1][r]), int(g[2][r])) == want, \
                            (vocab, k, targets, dr, a, want)
                for a, b in zip(same, real):
                    assert torch.equal(a, b), (vocab, k, targets)
                none = o.greedy_verify_logits(xx, vocab, d, accept=[-1] * n_req)
                for a, b in zip(none, real):
                    assert torch.equal(a, b), (vocab, k, targets)
    rng = random.Random(7)
    for trial in range(200):
        vocab = rng.randint(1, 4)
        n_req = rng.randint(1, 6)
        ks = [rng.randint(0, 4) for _ in range(n_req)]
        cu = [0]
        for k in ks:
            cu.append(cu[-1] + k)
        targets = [rng.randrange(vocab) for _ in range(cu[-1] + n_req)]
        drafts = [rng.randint(-1, vocab - 1) for _ in range(cu[-1])]
        acc = [rng.randint(-2, 5) for _ in range(n_req)]
        pf = [int(rng.random() < 0.3) for _ in range(n_req)] if trial % 2 else None
        x = _ragged_logits(targets, vocab)
        cu_t = torch.tensor(cu, dtype=torch.int32)
        d = torch.tensor(drafts, dtype=torch.int32)
        out, ns, nr, tg = o.greedy_verify_ragged(x, vocab, cu_t, d, prefilling=pf, accept=acc)
        assert tg.tolist() == targets
        for r, k in enumerate(ks):
            base = cu[r] + r
            got = (out[base:base + k + 1].tolist(), int(ns[r]), int(nr[r]))
            if pf and pf[r]:
                assert got == ([-1] * (k + 1), 0, 0), (cu, r, acc, got)
                continue
            want = bf.bf_verify_synthetic(targets[base:base + k + 1], drafts[cu[r]:cu[r] + k],
                                          acc[r])
            assert got == want, (cu, r, acc, got, want)


ALL_PINS = [pin_golden_argmax, pin_golden_block_stats, pin_golden_verify, pin_exhaustive_argmax,
            pin_torch_argmax, pin_slots, pin_block_stats_bruteforce, pin_invariance,
            pin_verify_bruteforce, pin_golden_epilogue, pin_scale_matches_torch,
            pin_ragged_verify, pin_synthetic_verify]
