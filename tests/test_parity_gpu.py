"""GPU parity: every output of the HIP path (statistics, token ids, value bits,
verification outputs) must equal the CPU oracle's bit for bit, on the same
seeded inputs.  The inputs are generated on the CPU (workloads.py), copied to
the device for the HIP path, and handed unchanged to the oracle."""
import ctypes
import random

import pytest
import torch

import oracle
import oracle_pins
import vocab_argmax_amd as vpa
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _announce(msg):
    print(f"[parity] {msg}", flush=True)


def _dev(x):
    return x.to(DEV)


def _host(x):
    torch.cuda.synchronize()
    return x.cpu()


def assert_same(got, want, what):
    got = _host(got)
    if not torch.equal(got, want):
        bad = (got != want).nonzero()
        raise AssertionError(f"{what}: {bad.shape[0]} mismatches, first at {bad[:4].tolist()}")


def check_stats_and_ids(x_cpu, vocab, w, s, block, name):
    """block_stats (all shards, then rank by rank), combine and top_tokens."""
    _announce(f"{name} block={block}")
    x = _dev(x_cpu)
    want_stats = oracle.block_stats(x_cpu, vocab, w, s, block)
    want_ids, want_vals = oracle.argmax(x_cpu, vocab)
    st = vpa.block_stats(x, vocab, w, s, block)
    assert_same(st, want_stats, f"{name} stats B={block}")
    ids, vals = vpa.combine_stats(st)
    assert_same(ids, want_ids, f"{name} combine ids")
    assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_vals, f"{name} combine vals")
    ids, vals = vpa.top_tokens(x, vocab, w, s, block)
    assert_same(ids, want_ids, f"{name} top_tokens ids")
    assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_vals, f"{name} top_tokens vals")
    # each rank reduces only its own columns (global ids, global block edges)
    parts = []
    for r in range(s):
        xr = x[:, r * w:min((r + 1) * w, x.shape[1])]
        parts.append(vpa.block_stats(xr, vocab, w, s, block, first_shard=r, n_local=1))
    assert_same(torch.cat(parts, 0), want_stats, f"{name} rank-wise stats")


def test_config1_argmax_v1000_fp32():
    w = workloads.config1()
    check_stats_and_ids(w.logits, w.vocab, w.shard_width, w.n_shards, 256, w.name)
    ids, _ = vpa.top_tokens(_dev(w.logits), w.vocab, w.shard_width, w.n_shards, 256)
    assert _host(ids)[[1, 3]].tolist() == [17, 17]


@pytest.mark.parametrize("case", workloads.edge_cases(), ids=lambda c: c.name)
def test_edge_cases(case):
    for b in case.blocks:
        check_stats_and_ids(case.logits, case.vocab, case.shard_width, case.n_shards, b, case.name)


def _verify_both(x_cpu, vocab, w, s, n_req, k, drafts, bd, bb, name):
    _announce(f"{name} verify R={n_req} K={k} blocks={bd}/{bb}")
    x = _dev(x_cpu)
    draft_rows, bonus_rows = oracle.verify_rows(n_req, k)
    want_d = oracle.block_stats(x_cpu, vocab, w, s, bd, rows=draft_rows)
    want_b = oracle.block_stats(x_cpu, vocab, w, s, bb, rows=bonus_rows)
    dst, bst = vpa.verify_stats(x, vocab, w, s, n_req, k, bd, bb)
    assert_same(dst, want_d, f"{name} draft stats")
    assert_same(bst, want_b, f"{name} bonus stats")
    want = oracle.greedy_verify(want_d, want_b, drafts)
    want_logits = oracle.greedy_verify_logits(x_cpu, vocab, drafts)
    for a, b in zip(want, want_logits):
        assert torch.equal(a, b)
    got = vpa.greedy_verify(dst, bst, _dev(drafts))
    for g, wv, nm in zip(got, want, ("out_tokens", "num_sampled", "num_rejected", "target_ids")):
        assert_same(g, wv, f"{name} {nm}")
    got_nt = vpa.greedy_verify(dst, bst, _dev(drafts), with_targets=False)
    for g, wv in zip(got_nt[:3], want[:3]):
        assert_same(g, wv, f"{name} (no target_ids)")
    # block_stats with explicit row lists gives the same statistics
    assert_same(vpa.block_stats(x, vocab, w, s, bd, rows=_dev(draft_rows)), want_d, f"{name} rows")
    # synthetic acceptance: per-request counts (some -1, i.e. real acceptance)
    acc = workloads.synthetic_counts(n_req, k, seed=131 * n_req + k)
    want_s = oracle.greedy_verify(want_d, want_b, drafts, accept=acc)
    for a, b in zip(want_s, oracle.greedy_verify_logits(x_cpu, vocab, drafts, accept=acc)):
        assert torch.equal(a, b)
    got_s = vpa.greedy_verify(dst, bst, _dev(drafts), accept=_dev(acc))
    for g, wv, nm in zip(got_s, want_s, ("out_tokens", "num_sampled", "num_rejected",
                                         "target_ids")):
        assert_same(g, wv, f"{name} synthetic {nm}")
    return want


@pytest.mark.parametrize("case", workloads.edge_cases(), ids=lambda c: c.name)
def test_edge_verify(case):
    x, v, w, s = case.logits, case.vocab, case.shard_width, case.n_shards
    tgt, _ = oracle.argmax(x, v)
    for k in (1, 5):
        for plan, uniform in workloads.edge_verify_plans(k, v):
            n_req = plan.shape[0]
            targets = tgt[:n_req * (k + 1)].reshape(n_req, k + 1)
            drafts = workloads.compose_drafts(targets, plan, uniform)
            for bd, bb in ((8192, 1024), (256, 1000)):
                _verify_both(x, v, w, s, n_req, k, drafts, bd, bb, case.name)


@pytest.mark.parametrize("k", [2, 16, 17, 40])
def test_verify_many_drafts(k):
    """K beyond one wavefront per position (more positions than waves in the
    finishing workgroup), random plans including placeholders."""
    vocab, s = 1000, 3
    w = -(-vocab // s)
    n_req = 9
    g = torch.Generator().manual_seed(4000 + k)
    x = (torch.randn((n_req * (k + 1), s * w), generator=g) * 2).to(torch.bfloat16)
    x[:, vocab:] = float("nan")
    tgt, _ = oracle.argmax(x, vocab)
    plan = torch.where(torch.rand((n_req, k), generator=g) < 0.9, 1, 0).to(torch.int8)
    plan[0, k // 2:] = -1
    plan[1, :] = 1
    uniform = torch.randint(0, vocab, (n_req, k), generator=g, dtype=torch.int64).to(torch.int32)
    drafts = workloads.compose_drafts(tgt.reshape(n_req, k + 1), plan, uniform)
    _verify_both(x, vocab, w, s, n_req, k, drafts, 256, 64, f"many drafts K={k}")


def test_verify_at_the_draft_limit():
    """K = VPA_MAX_DRAFTS (4096), uniform and ragged: one request with every
    draft accepted (bonus token at position K), one rejected deep inside;
    a ragged batch with a 4096-draft request, a zero-draft request and a
    request still prefilling."""
    k, vocab, s = 4096, 50, 2
    w = vocab // s
    n_req = 2
    g = torch.Generator().manual_seed(4096)
    x = (torch.randn((n_req * (k + 1), s * w), generator=g) * 2).to(torch.bfloat16)
    tgt, _ = oracle.argmax(x, vocab)
    targets = tgt.reshape(n_req, k + 1)
    plan = torch.ones((n_req, k), dtype=torch.int8)
    plan[1, 3000] = 0
    uniform = torch.zeros((n_req, k), dtype=torch.int32)
    uniform[1, 3000] = (int(targets[1, 3000]) + 1) % vocab      # a sure mismatch
    drafts = workloads.compose_drafts(targets, plan, uniform)
    want = _verify_both(x, vocab, w, s, n_req, k, drafts, 256, 16, "draft limit")
    assert want[1].tolist() == [k + 1, 3001]
    # ragged: K_r = 4096, 0, 5; the last request is still prefilling
    cu = torch.tensor([0, k, k, k + 5], dtype=torch.int32)
    total = int(cu[-1])
    xr = (torch.randn((total + 3, s * w), generator=g) * 2).to(torch.bfloat16)
    tr, _ = oracle.argmax(xr, vocab)
    draft_rows, _ = oracle.ragged_rows(cu)
    dr = tr[draft_rows.long()].to(torch.int32)
    dr[1234] = (int(dr[1234]) + 1) % vocab
    pf = torch.tensor([0, 0, 1], dtype=torch.uint8)
    _announce(f"ragged draft limit total={total}")
    want_r = oracle.greedy_verify_ragged(xr, vocab, cu, dr, prefilling=pf)
    got_r = vpa.verify_ragged(_dev(xr), vocab, w, s, _dev(cu), _dev(dr), total,
                              prefilling=_dev(pf))
    for a, b, nm in zip(got_r, want_r, ("out_tokens", "num_sampled", "num_rejected",
                                        "target_ids")):
        assert_same(a, b, f"ragged draft limit {nm}")
    assert want_r[1].tolist() == [1235, 1, 0]
    # synthetic counts at the limit: all 4096 drafts accepted past the planted
    # mismatch, a count above K_r = 0, and a prefilling request's count ignored
    acc = torch.tensor([k, 7, 2], dtype=torch.int32)
    want_a = oracle.greedy_verify_ragged(xr, vocab, cu, dr, prefilling=pf, accept=acc)
    got_a = vpa.verify_ragged(_dev(xr), vocab, w, s, _dev(cu), _dev(dr), total,
                              prefilling=_dev(pf), accept=_dev(acc))
    for a, b, nm in zip(got_a, want_a, ("out_tokens", "num_sampled", "num_rejected",
                                        "target_ids")):
        assert_same(a, b, f"ragged draft limit synthetic {nm}")
    assert want_a[1].tolist() == [k + 1, 1, 0]


def test_one_column_shards_and_more_shards_than_columns():
    """Degenerate shard geometries: one column per shard (S = V = 1000,
    W = 1), and more shards than valid columns (S = 1500, W = 1: shards past
    V hold only padding and give empty statistics), at blocks of 1, 7 and
    8192 columns, in both dtypes."""
    for dtype in (torch.bfloat16, torch.float32):
        for vocab, s in ((1000, 1000), (1000, 1500)):
            x_cpu = oracle_pins._special_matrix(5, s, 7000 + s, dtype)
            x_cpu[:, vocab:] = float("nan")
            x = _dev(x_cpu)
            want_ids, want_vals = oracle.argmax(x_cpu, vocab)
            for block in (1, 7, 8192):
                name = f"one-column shards V={vocab} S={s} B={block} {dtype}"
                _announce(name)
                assert_same(vpa.block_stats(x, vocab, 1, s, block),
                            oracle.block_stats(x_cpu, vocab, 1, s, block), name)
                ids, vals = vpa.top_tokens(x, vocab, 1, s, block)
                assert_same(ids, want_ids, name + " ids")
                assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_vals, name + " vals")


@pytest.mark.parametrize("scale", [1.0, 0.7, 1 / 0.7, 1e-40, 3e38])
def test_epilogue_d2t_and_scale(scale):
    """top_tokens and combine_stats with a draft-to-target table and a positive
    scale: ids unchanged, maxima scaled in fp32 (round to nearest, subnormals
    kept, NaN untouched, overflow to inf), mapped ids = k + d2t[k]."""
    cases = [workloads.config2(), workloads.edge_cases()[0], workloads.edge_cases()[3]]
    for w in cases:
        _announce(f"epilogue {w.name} scale={scale}")
        x_cpu, v = w.logits, w.vocab
        g = torch.Generator().manual_seed(v)
        d2t = torch.randint(-100, 100000, (v + 3,), generator=g, dtype=torch.int64)
        want_ids, want_vals = oracle.argmax(x_cpu, v)
        want_scaled = oracle.scale_bits(want_vals, scale)
        want_mapped = oracle.map_ids(want_ids, d2t)
        x, dd = _dev(x_cpu), _dev(d2t)
        block = w.blocks[0]
        ids, vals, mapped = vpa.top_tokens(x, v, w.shard_width, w.n_shards, block, d2t=dd,
                                           scale=scale)
        assert_same(ids, want_ids, "epilogue ids")
        assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_scaled, "epilogue scaled values")
        assert_same(mapped, want_mapped, "epilogue mapped ids")
        ids2, vals2 = vpa.top_tokens(x, v, w.shard_width, w.n_shards, block, scale=scale)
        assert_same(vals2.to(torch.int64) & 0xFFFFFFFF, want_scaled, "scale only")
        st = vpa.block_stats(x, v, w.shard_width, w.n_shards, block)
        ids3, vals3, mapped3 = vpa.combine_stats(st, d2t=dd, scale=scale)
        assert_same(ids3, want_ids, "combine epilogue ids")
        assert_same(vals3.to(torch.int64) & 0xFFFFFFFF, want_scaled, "combine scaled values")
        assert_same(mapped3, want_mapped, "combine mapped ids")


def test_epilogue_short_table_maps_outside_ids_to_minus_one():
    """combine_stats accepts any table length; ids past it map to -1."""
    w = workloads.config1()
    x_cpu = w.logits
    want_ids, _ = oracle.argmax(x_cpu, w.vocab)
    d2t = torch.arange(20, dtype=torch.int64) * 3          # covers ids 0..19 only
    st = vpa.block_stats(_dev(x_cpu), w.vocab, w.shard_width, w.n_shards, 256)
    ids, vals, mapped = vpa.combine_stats(st, d2t=_dev(d2t))
    assert_same(mapped, oracle.map_ids(want_ids, d2t), "short table")


def _ragged_case(seed, vocab, s, n_req, kmax, dtype=torch.bfloat16, p_copy=0.7):
    g = torch.Generator().manual_seed(seed)
    ks = torch.randint(0, kmax + 1, (n_req,), generator=g)
    cu = torch.zeros(n_req + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(ks, 0).to(torch.int32)
    total = int(cu[-1])
    w = -(-vocab // s)
    x = (torch.randn((total + n_req, s * w), generator=g) * 3).to(dtype)
    x[:, vocab:] = float("nan")
    tgt, _ = oracle.argmax(x, vocab)
    draft_rows, _ = oracle.ragged_rows(cu)
    plan = torch.where(torch.rand(total, generator=g) < p_copy, 1, 0)
    plan = torch.where(torch.rand(total, generator=g) < 0.05, -1, plan)
    uni = torch.randint(0, vocab, (total,), generator=g, dtype=torch.int64).to(torch.int32)
    drafts = workloads.compose_drafts(tgt[draft_rows.long()][None, :], plan[None, :].to(torch.int8),
                                      uni[None, :])[0]
    return x, vocab, w, s, cu, drafts


@pytest.mark.parametrize("seed,vocab,s,n_req,kmax", [(1, 1000, 3, 7, 4), (2, 50257, 3, 13, 6),
                                                     (3, 200064, 4, 24, 5), (4, 997, 8, 40, 0),
                                                     (5, 2000, 2, 1, 40)])
def test_ragged_verify(seed, vocab, s, n_req, kmax):
    """Per-request draft counts (some zero): row lists, one statistics launch for
    both row lists, and the ragged finish, against the oracle."""
    x_cpu, v, w, s, cu, drafts = _ragged_case(seed, vocab, s, n_req, kmax)
    _announce(f"ragged V={v} S={s} R={n_req} Kmax={kmax} total={int(cu[-1])}")
    want = oracle.greedy_verify_ragged(x_cpu, v, cu, drafts)
    draft_rows, bonus_rows = oracle.ragged_rows(cu)
    want_d = oracle.block_stats(x_cpu, v, w, s, 8192, rows=draft_rows)
    want_b = oracle.block_stats(x_cpu, v, w, s, 1024, rows=bonus_rows)
    want_s = oracle.greedy_verify_ragged_stats(want_d, want_b, cu, drafts)
    for a, b in zip(want, want_s):
        assert torch.equal(a, b)
    x, cud, dd = _dev(x_cpu), _dev(cu), _dev(drafts)
    total = int(cu[-1])
    dr, br = vpa.ragged_rows(cud, total)
    assert_same(dr, draft_rows, "draft rows")
    assert_same(br, bonus_rows, "bonus rows")
    dst, bst = vpa.verify_stats_rows(x, v, w, s, dr, br, 8192, 1024)
    assert_same(dst, want_d, "ragged draft stats")
    assert_same(bst, want_b, "ragged bonus stats")
    got = vpa.greedy_verify_ragged(dst, bst, cud, dd, total)
    for g, wv, nm in zip(got, want, ("out_tokens", "num_sampled", "num_rejected", "target_ids")):
        assert_same(g, wv, f"ragged {nm}")
    got2 = vpa.verify_ragged(x, v, w, s, cud, dd, total, with_targets=False)
    for g, wv in zip(got2[:3], want[:3]):
        assert_same(g, wv, "verify_ragged")
    # about a third of the requests still prefilling (they sample nothing)
    pf = torch.rand(n_req, generator=torch.Generator().manual_seed(seed + 50)) < 0.35
    want_p = oracle.greedy_verify_ragged(x_cpu, v, cu, drafts, prefilling=pf)
    got_p = vpa.greedy_verify_ragged(dst, bst, cud, dd, total, prefilling=_dev(pf))
    for g, wv, nm in zip(got_p, want_p, ("out_tokens", "num_sampled", "num_rejected",
                                         "target_ids")):
        assert_same(g, wv, f"ragged prefilling {nm}")
    got_p2 = vpa.verify_ragged(x, v, w, s, cud, dd, total, with_targets=False,
                               prefilling=_dev(pf.to(torch.uint8)))
    for g, wv in zip(got_p2[:3], want_p[:3]):
        assert_same(g, wv, "verify_ragged prefilling")
    # synthetic accept counts, alone and together with the prefilling flags
    acc = workloads.synthetic_counts(n_req, kmax, seed=seed + 70)
    for flags in (None, pf):
        want_a = oracle.greedy_verify_ragged(x_cpu, v, cu, drafts, prefilling=flags, accept=acc)
        got_a = vpa.greedy_verify_ragged(dst, bst, cud, dd, total,
                                         prefilling=None if flags is None else _dev(flags),
                                         accept=_dev(acc))
        for g, wv, nm in zip(got_a, want_a, ("out_tokens", "num_sampled", "num_rejected",
                                             "target_ids")):
            assert_same(g, wv, f"ragged synthetic {nm} prefilling={flags is not None}")


def test_random_ragged_batches():
    """30 random ragged batches (draft counts 0..K_max per request, both
    dtypes, several vocabularies and shard counts): the whole ragged path
    against the oracle's ragged verification from full logits."""
    rng = random.Random(31)
    for trial in range(30):
        vocab = rng.choice([5, 1000, 4097, 50257])
        s = rng.choice([1, 2, 3, 8])
        n_req = rng.choice([1, 3, 17, 64])
        kmax = rng.choice([0, 1, 4, 9])
        dtype = torch.float32 if trial % 3 == 0 else torch.bfloat16
        x_cpu, v, w, s, cu, drafts = _ragged_case(100 + trial, vocab, s, n_req, kmax, dtype,
                                                  p_copy=rng.random())
        total = int(cu[-1])
        pf = None
        if trial % 2:
            pf = torch.tensor([rng.random() < 0.3 for _ in range(n_req)], dtype=torch.bool)
        acc = workloads.synthetic_counts(n_req, kmax, seed=500 + trial) if trial % 3 == 1 else None
        _announce(f"random ragged {trial} V={v} S={s} R={n_req} Kmax={kmax} total={total} {dtype}"
                  f" prefilling={None if pf is None else int(pf.sum())} synthetic={acc is not None}")
        want = oracle.greedy_verify_ragged(x_cpu, v, cu, drafts, prefilling=pf, accept=acc)
        got = vpa.verify_ragged(_dev(x_cpu), v, w, s, _dev(cu), _dev(drafts), total,
                                prefilling=None if pf is None else _dev(pf),
                                accept=None if acc is None else _dev(acc))
        for a, b, nm in zip(got, want, ("out_tokens", "num_sampled", "num_rejected", "target_ids")):
            assert_same(a, b, f"random ragged {trial} {nm}")


def test_ragged_malformed_offsets_are_flagged():
    """Offsets that decrease or run past the total: that request reports -1
    counts and writes no tokens; the others are unaffected."""
    x_cpu, v, w, s, cu, drafts = _ragged_case(9, 1000, 2, 4, 3)
    total = int(cu[-1])
    bad = cu.clone()
    bad[2] = total + 50                      # request 1 runs past, request 2 decreases
    dst = vpa.block_stats(_dev(x_cpu), v, w, s, 8192, rows=_dev(torch.arange(total, dtype=torch.int32)))
    bst = vpa.block_stats(_dev(x_cpu), v, w, s, 1024,
                          rows=_dev(torch.arange(4, dtype=torch.int32)))
    out, ns, nr, tg = vpa.greedy_verify_ragged(dst, bst, _dev(bad), _dev(drafts), total)
    ns, nr = _host(ns), _host(nr)
    assert ns[1] == -1 and nr[1] == -1 and ns[2] == -1 and nr[2] == -1
    assert ns[0] >= 1 and ns[3] >= 1
    dr, br = vpa.ragged_rows(_dev(bad), total)
    assert _host(br)[1:3].tolist() == [-1, -1]
    # malformed offsets win over a prefilling flag; a prefilling request
    # with good offsets samples nothing
    pf = _dev(torch.tensor([1, 1, 0, 0], dtype=torch.uint8))
    out, ns, nr, tg = vpa.greedy_verify_ragged(dst, bst, _dev(bad), _dev(drafts), total,
                                               prefilling=pf)
    ns, nr, out = _host(ns), _host(nr), _host(out)
    assert ns[:3].tolist() == [0, -1, -1] and nr[:3].tolist() == [0, -1, -1]
    k0 = int(cu[1])
    assert out[:k0 + 1].tolist() == [-1] * (k0 + 1)
    assert ns[3] >= 1


def test_row_list_out_of_range_rows_are_empty():
    case = workloads.edge_cases()[3]                      # vocab 1000, 8 shards, bf16
    x = _dev(case.logits)
    rows = torch.tensor([3, 0, -1, 16, 15, 1 << 30], dtype=torch.int32)
    st = _host(vpa.block_stats(x, case.vocab, case.shard_width, case.n_shards, 256, rows=_dev(rows)))
    want = oracle.block_stats(case.logits, case.vocab, case.shard_width, case.n_shards, 256,
                              rows=torch.tensor([3, 0, 15]))
    assert torch.equal(st[:, [0, 1, 4]], want)
    for i in (2, 3, 5):
        assert bool((st[:, i, :, 0] == torch.tensor(vpa.EMPTY_BITS).to(torch.int32)).all())
        assert bool((st[:, i, :, 1] == vpa.EMPTY_ID).all())


def _random_case(rng, trial):
    """A padded [rows, S*W + pad] matrix and a column offset `off` <= pad: the
    case is the view full[:, off:], whose base is misaligned by `off` elements
    and whose valid columns stay inside the buffer."""
    dtype = torch.float32 if trial % 2 else torch.bfloat16
    s = rng.choice([1, 2, 3, 4, 5, 8])
    vocab = rng.choice([1, 2, 7, 63, 1000, 4097, 50257, 70001])
    w = -(-vocab // s) + rng.choice([0, 0, 1, 3, 64])
    block = rng.choice([1, 3, 64, 255, 256, 1000, 1024, 8192, 65536, 1 << 20])
    if vocab > 10000 and block < 64:
        block = 64
    pad = rng.choice([0, 1, 5, 8])
    off = rng.randint(0, pad)
    n_rows = rng.choice([1, 3, 9])
    full = oracle_pins._special_matrix(n_rows, s * w + pad, 9000 + trial, dtype)
    full[:, vocab:s * w] = float("nan")
    return full, off, vocab, w, s, block


def test_draft_model_vocab_40960_k15():
    """The smallest vocabulary the pages name (40960, a draft model's, in
    PR #39419, "Current Issue") at TP2 and TP4, with K = 15 drafts per
    request as in their DFlash runs: statistics, argmax and verification."""
    v = 40960
    g = torch.Generator().manual_seed(40960)
    x = (torch.randn((64, v), generator=g) * 3).to(torch.bfloat16)
    x[3, 20479] = 30.0                        # a tie across the TP2 shard edge
    x[3, 20480] = 30.0
    for s in (2, 4):
        w = v // s
        for block in (8192, 1024):
            check_stats_and_ids(x, v, w, s, block, f"V=40960 S={s}")
        n_req, k = 4, 15
        tgt, _ = oracle.argmax(x, v)
        plan = (torch.rand((n_req, k), generator=g) < 0.8).to(torch.int8)
        drafts = workloads.compose_drafts(tgt.reshape(n_req, k + 1), plan,
                                          torch.randint(0, v, (n_req, k), generator=g,
                                                        dtype=torch.int64).to(torch.int32))
        _verify_both(x, v, w, s, n_req, k, drafts, 8192, 1024, f"V=40960 S={s} K=15")
    assert int(_host(vpa.top_tokens(_dev(x), v, v // 2, 2, 8192)[0])[3]) == 20479


def test_random_geometries():
    """Random V, S, W, block, dtype, row padding and base misalignment."""
    rng = random.Random(1234)
    for trial in range(80):
        full, off, vocab, w, s, block = _random_case(rng, trial)
        x_cpu = full[:, off:]
        x = _dev(full)[:, off:]
        name = f"random{trial} V={vocab} S={s} W={w} B={block} ld={full.shape[1]} off={off} {full.dtype}"
        _announce(name)
        want_stats = oracle.block_stats(x_cpu, vocab, w, s, block)
        assert_same(vpa.block_stats(x, vocab, w, s, block), want_stats, name)
        want_ids, want_vals = oracle.argmax(x_cpu, vocab)
        ids, vals = vpa.top_tokens(x, vocab, w, s, block)
        assert_same(ids, want_ids, name + " ids")
        assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_vals, name + " vals")


def test_random_verification_geometries():
    """Random V, S, W, K, request count, block pair and dtype, with special
    values in the logits and drafts that copy the target, draw uniformly,
    or are placeholders: verification statistics and the greedy finish
    against the oracle (which also checks them against full-row argmax)."""
    rng = random.Random(777)
    for trial in range(40):
        dtype = torch.float32 if trial % 2 else torch.bfloat16
        s = rng.choice([1, 2, 3, 4, 8])
        vocab = rng.choice([2, 63, 1000, 4097, 50257])
        w = -(-vocab // s) + rng.choice([0, 1, 64])
        k = rng.choice([1, 2, 3, 5, 7, 15])
        n_req = rng.choice([1, 2, 5, 13])
        bd, bb = rng.choice([(8192, 1024), (1024, 256), (256, 64), (4096, 8192), (1 << 20, 1)])
        if vocab > 10000 and min(bd, bb) < 64:
            bd, bb = 8192, 1024
        rows = n_req * (k + 1) + rng.choice([0, 3])
        x = oracle_pins._special_matrix(rows, s * w, 7000 + trial, dtype)
        x[:, vocab:] = float("nan")
        tgt, _ = oracle.argmax(x, vocab)
        g = torch.Generator().manual_seed(7000 + trial)
        plan = torch.randint(-1, 2, (n_req, k), generator=g).to(torch.int8)
        uni = torch.randint(0, vocab, (n_req, k), generator=g, dtype=torch.int64).to(torch.int32)
        drafts = workloads.compose_drafts(tgt[:n_req * (k + 1)].reshape(n_req, k + 1), plan, uni)
        _verify_both(x, vocab, w, s, n_req, k, drafts, bd, bb,
                     f"random verify {trial} V={vocab} S={s} W={w} K={k} R={n_req} B={bd}/{bb} {dtype}")


def test_long_segments_and_chunk_cascade():
    """Blocks far larger than one pipelined chunk (many chunks per segment),
    segments that end part-way through a chunk, and ties planted far
    apart."""
    for dtype in (torch.bfloat16, torch.float32):
        for vocab, s, block in ((200064, 2, 1 << 20), (200064, 1, 1 << 21), (131071, 3, 65536),
                                (9000, 1, 9000), (5000, 1, 4608)):
            w = -(-vocab // s)
            g = torch.Generator().manual_seed(vocab + s)
            x = (torch.randn((4, s * w), generator=g) * 3).to(dtype)
            x[:, vocab:] = float("nan")
            x[1, 5] = 100.0
            x[1, vocab - 3] = 100.0
            x[2, vocab // 2] = float("nan")
            x[2, vocab - 1] = float("nan")
            x[3, :vocab] = float("-inf")
            check_stats_and_ids(x, vocab, w, s, block, f"long V={vocab} S={s} B={block} {dtype}")


def test_largest_vocabulary():
    """V = 2^24 - 1, the largest the boundary accepts, over 8 shards of
    2^21 columns: ids up to 2^24 - 2, one padding column, both dtypes and
    both block sizes of the pages."""
    v, s = (1 << 24) - 1, 8
    w = -(-v // s)
    for dtype in (torch.bfloat16, torch.float32):
        g = torch.Generator().manual_seed(24)
        x = (torch.randn((3, s * w), generator=g) * 3).to(dtype)
        x[:, v:] = float("inf")
        x[0, v - 1] = 50.0
        x[1, v - 1] = float("nan")
        x[2, 0] = 50.0
        x[2, v - 1] = 50.0
        for block in (8192, 1024):
            check_stats_and_ids(x, v, w, s, block, f"V=2^24-1 {dtype}")
        ids, _ = vpa.top_tokens(_dev(x), v, w, s, 8192)
        assert _host(ids).tolist() == [v - 1, v - 1, 0]


def test_config2_top_tokens_v151936_bf16_tp2():
    w = workloads.config2()
    check_stats_and_ids(w.logits, w.vocab, w.shard_width, w.n_shards, 8192, w.name)


def test_config3_verify_v200064_bf16_tp4():
    w = workloads.config3()
    tgt, _ = oracle.argmax(w.logits, w.vocab)
    drafts = workloads.compose_drafts(tgt.reshape(w.n_req, w.k + 1), w.draft_plan, w.draft_uniform)
    want = _verify_both(w.logits, w.vocab, w.shard_width, w.n_shards, w.n_req, w.k, drafts, 8192,
                        1024, w.name)
    # the plan copies the target with p=0.7: some but not all drafts accepted
    assert 0 < int(want[2].sum()) < w.n_req * w.k


def test_config4_full_size_4096_rows():
    """4096 x 200064 bf16 at 8 shards, in the launch shapes the benchmark times."""
    w = workloads.config4()
    _announce(f"{w.name}: oracle argmax")
    want_ids, want_vals = oracle.argmax(w.logits, w.vocab)
    x = _dev(w.logits)
    ids, vals = vpa.top_tokens(x, w.vocab, w.shard_width, w.n_shards, 8192)
    assert_same(ids, want_ids, "config4 ids")
    assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_vals, "config4 vals")
    _announce(f"{w.name}: oracle block stats")
    want_stats = oracle.block_stats(w.logits, w.vocab, w.shard_width, w.n_shards, 8192)
    assert_same(vpa.block_stats(x, w.vocab, w.shard_width, w.n_shards, 8192), want_stats, "config4 stats")
    drafts = workloads.compose_drafts(want_ids[:w.n_req * (w.k + 1)].reshape(w.n_req, w.k + 1),
                                      w.draft_plan, w.draft_uniform)
    _verify_both(w.logits, w.vocab, w.shard_width, w.n_shards, w.n_req, w.k, drafts, 8192, 1024,
                 w.name)

    # the epilogue call the benchmark times: a 200064-entry table, scale 1/0.7
    _announce(f"{w.name}: epilogue")
    g = torch.Generator().manual_seed(4004)
    d2t = torch.randint(0, 1000, (w.vocab,), generator=g, dtype=torch.int64)
    ids, vals, mapped = vpa.top_tokens(x, w.vocab, w.shard_width, w.n_shards, 8192, d2t=_dev(d2t),
                                       scale=1 / 0.7)
    assert_same(ids, want_ids, "config4 epilogue ids")
    assert_same(vals.to(torch.int64) & 0xFFFFFFFF, oracle.scale_bits(want_vals, 1 / 0.7),
                "config4 epilogue values")
    assert_same(mapped, oracle.map_ids(want_ids, d2t), "config4 epilogue mapped ids")

    # the ragged batch the benchmark times: K_r = 7r mod 11 drafts over 682
    # requests (3410 drafts, rows 0..4091), drafts copying their target with p = 1/2
    _announce(f"{w.name}: ragged verification")
    ks = [(7 * r) % 11 for r in range(w.n_req)]
    cu = torch.tensor([0] + [sum(ks[:r + 1]) for r in range(w.n_req)], dtype=torch.int32)
    total = int(cu[-1])
    tgt = torch.cat([want_ids[int(cu[r]) + r:int(cu[r + 1]) + r] for r in range(w.n_req)])
    keep = torch.rand(total, generator=g) < 0.5
    drafts_r = torch.where(keep, tgt, torch.randint(0, w.vocab, (total,), generator=g,
                                                    dtype=torch.int64).to(torch.int32))
    want = oracle.greedy_verify_ragged(w.logits, w.vocab, cu, drafts_r)
    got = vpa.verify_ragged(x, w.vocab, w.shard_width, w.n_shards, _dev(cu), _dev(drafts_r), total)
    for a, b, nm in zip(got, want, ("out_tokens", "num_sampled", "num_rejected", "target_ids")):
        assert_same(a, b, f"config4 ragged {nm}")
    _announce(f"{w.name}: ragged verification, synthetic acceptance")
    acc = workloads.synthetic_counts(w.n_req, 10, seed=4005)
    want = oracle.greedy_verify_ragged(w.logits, w.vocab, cu, drafts_r, accept=acc)
    got = vpa.verify_ragged(x, w.vocab, w.shard_width, w.n_shards, _dev(cu), _dev(drafts_r), total,
                            accept=_dev(acc))
    for a, b, nm in zip(got, want, ("out_tokens", "num_sampled", "num_rejected", "target_ids")):
        assert_same(a, b, f"config4 ragged synthetic {nm}")


def test_fp32_1024_rows_full_vocab():
    """fp32 at scale: 1024 x 200064 fp32 (0.8 GB), 8 shards, top_tokens and the
    verification statistics, every output against the oracle."""
    g = torch.Generator().manual_seed(77)
    v, w, s = 200064, 25008, 8
    x_cpu = torch.randn((1024, v), generator=g) * 3
    x_cpu[7, 199999] = float("nan")
    x_cpu[9, :] = float("-inf")
    x_cpu[11, 25007] = 50.0
    x_cpu[11, 25008] = 50.0
    _announce("fp32 1024 x 200064")
    want_ids, want_vals = oracle.argmax(x_cpu, v)
    x = _dev(x_cpu)
    ids, vals = vpa.top_tokens(x, v, w, s, 8192)
    assert_same(ids, want_ids, "fp32 ids")
    assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_vals, "fp32 vals")
    assert int(_host(ids)[11]) == 25007
    n_req, k = 170, 5
    plan = torch.ones((n_req, k), dtype=torch.int8)
    plan[::3, 2] = 0
    uni = torch.zeros((n_req, k), dtype=torch.int32)
    drafts = workloads.compose_drafts(want_ids[:n_req * (k + 1)].reshape(n_req, k + 1), plan, uni)
    _verify_both(x_cpu, v, w, s, n_req, k, drafts, 8192, 1024, "fp32 verify")


def test_row_offsets_beyond_4gb():
    """64-bit addressing: rows 1.2e9 elements apart (2.4 GB of bf16), so row 2
    starts 4.8 GB into the buffer, past 2^31 elements and 2^32 bytes.  Only
    the first V columns of each row are filled and read."""
    v, w, s, ld = 200064, 25008, 8, 1_200_000_000
    g = torch.Generator().manual_seed(4096)
    x_cpu = (torch.randn((3, v), generator=g) * 3).to(torch.bfloat16)
    x_cpu[2, 199_000] = 40.0
    x_cpu[1, 5] = float("nan")
    _announce("3 rows, ld = 1.2e9 (7.2 GB buffer)")
    big = torch.empty((3, ld), dtype=torch.bfloat16, device=DEV)
    big[:, :v] = _dev(x_cpu)
    x = big[:, :v]
    assert x.stride(0) == ld
    want_ids, want_vals = oracle.argmax(x_cpu, v)
    ids, vals = vpa.top_tokens(x, v, w, s, 8192)
    assert_same(ids, want_ids, "ids beyond 4 GB")
    assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_vals, "vals beyond 4 GB")
    assert _host(ids).tolist()[1:] == [5, 199_000]
    rows = torch.tensor([2, 0, 2, 1], dtype=torch.int32)
    st = vpa.block_stats(x, v, w, s, 1024, rows=_dev(rows))
    assert_same(st, oracle.block_stats(x_cpu, v, w, s, 1024, rows=rows), "row-list stats")
    drafts = torch.tensor([[int(want_ids[0]), 7]], dtype=torch.int32)
    got = vpa.greedy_verify(*vpa.verify_stats(x, v, w, s, 1, 2), _dev(drafts))
    for a, b in zip(got, oracle.greedy_verify_logits(x_cpu, v, drafts)):
        assert_same(a, b, "verification beyond 4 GB")
    del big, x
    torch.cuda.empty_cache()


def test_repeat_runs_are_bitwise_identical():
    w = workloads.config2()
    x = _dev(w.logits)
    first = [t.clone() for t in vpa.top_tokens(x, w.vocab, w.shard_width, w.n_shards, 8192)]
    st0 = vpa.block_stats(x, w.vocab, w.shard_width, w.n_shards, 1024).clone()
    for _ in range(5):
        again = vpa.top_tokens(x, w.vocab, w.shard_width, w.n_shards, 8192)
        for a, b in zip(first, again):
            assert torch.equal(a, b)
        assert torch.equal(st0, vpa.block_stats(x, w.vocab, w.shard_width, w.n_shards, 1024))


def test_top_tokens_workspace_reused_across_shapes():
    """One workspace, filled with garbage once, serves calls of different
    shapes, dtypes and block sizes in a row: its contents on entry do not
    matter, and each call's outputs equal the oracle's."""
    cases = [(c.logits, c.vocab, c.shard_width, c.n_shards, b, c.name)
             for c in workloads.edge_cases()[:3] for b in c.blocks]
    w2 = workloads.config2()
    cases.insert(2, (w2.logits, w2.vocab, w2.shard_width, w2.n_shards, 8192, w2.name))
    need = max(vpa.top_tokens_workspace(v, wd, s, x.shape[0], b) for x, v, wd, s, b, _ in cases)
    g = torch.Generator().manual_seed(91)
    ws = _dev(torch.randint(0, 256, (need,), generator=g, dtype=torch.int32).to(torch.uint8))
    for x_cpu, v, wd, s, b, name in cases:
        _announce(f"shared workspace: {name} block={b}")
        want_ids, want_vals = oracle.argmax(x_cpu, v)
        ids, vals = vpa.top_tokens(_dev(x_cpu), v, wd, s, b, workspace=ws)
        assert_same(ids, want_ids, f"{name} B={b} ids")
        assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_vals, f"{name} B={b} vals")


def test_top_tokens_rejects_bad_output_tensors():
    """Caller-supplied outputs are checked before any launch: wrong dtype,
    wrong length or a non-contiguous workspace raise, and nothing is written."""
    x = _dev(oracle_pins._special_matrix(4, 1000, 99, torch.bfloat16))
    n = 4
    good = dict(ids=torch.zeros(n, dtype=torch.int32, device=DEV),
                val_bits=torch.zeros(n, dtype=torch.int32, device=DEV))
    bad = [dict(ids=torch.zeros(n, dtype=torch.int64, device=DEV)),
           dict(ids=torch.zeros(n - 1, dtype=torch.int32, device=DEV)),
           dict(val_bits=torch.zeros(2 * n, dtype=torch.int32, device=DEV)[::2]),
           dict(d2t=torch.zeros(1000, dtype=torch.int64, device=DEV),
                mapped=torch.zeros(n, dtype=torch.int32, device=DEV)),
           dict(workspace=torch.zeros((2, 4096), dtype=torch.uint8, device=DEV)[:, ::2])]
    for kw in bad:
        args = dict(good)
        args.update(kw)
        with pytest.raises(ValueError):
            vpa.top_tokens(x, 1000, 250, 4, 256, **args)
    torch.cuda.synchronize()
    assert int(good["ids"].abs().sum()) == 0          # nothing was launched
    ids, _ = vpa.top_tokens(x, 1000, 250, 4, 256, **good)
    assert_same(ids, oracle.argmax(x.cpu(), 1000)[0], "good outputs")


def test_two_streams_run_concurrently():
    """The library keeps no device state between calls: two streams each run
    the draft argmax and the verification on their own data, interleaved
    call by call, and both match the oracle."""
    w = workloads.config3()
    v, wd, s, r, k = w.vocab, w.shard_width, w.n_shards, w.n_req, w.k
    g = torch.Generator().manual_seed(4242)
    xs = [w.logits, (torch.randn(w.logits.shape, generator=g) * 3).to(torch.bfloat16)]
    drafts = []
    for x_cpu in xs:
        tgt, _ = oracle.argmax(x_cpu, v)
        plan = (torch.rand((r, k), generator=g) < 0.5).to(torch.int8)
        drafts.append(workloads.compose_drafts(tgt.reshape(r, k + 1), plan,
                                               torch.zeros((r, k), dtype=torch.int32)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    xd = [_dev(x) for x in xs]
    dd = [_dev(d) for d in drafts]
    torch.cuda.synchronize()
    results = [[], []]
    for _ in range(3):
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                ids, vals = vpa.top_tokens(xd[i], v, wd, s, 8192)
                out = vpa.greedy_verify(*vpa.verify_stats(xd[i], v, wd, s, r, k), dd[i])
                results[i].append((ids, vals) + tuple(out))
    torch.cuda.synchronize()
    for i in (0, 1):
        _announce(f"stream {i}")
        want_ids, want_vals = oracle.argmax(xs[i], v)
        want = oracle.greedy_verify_logits(xs[i], v, drafts[i])
        for got in results[i]:
            assert_same(got[0], want_ids, f"stream {i} ids")
            assert_same(got[1].to(torch.int64) & 0xFFFFFFFF, want_vals, f"stream {i} vals")
            for a, b in zip(got[2:], want):
                assert_same(a, b, f"stream {i} verification")


def test_explicit_stream_argument():
    """Every call accepts an explicit torch stream: work enqueued on a side
    stream, synchronised on that stream alone, matches the oracle."""
    w = workloads.config3()
    v, wd, s, r, k = w.vocab, w.shard_width, w.n_shards, w.n_req, w.k
    x = _dev(w.logits)
    tgt, vals = oracle.argmax(w.logits, v)
    drafts = workloads.compose_drafts(tgt.reshape(r, k + 1), w.draft_plan, w.draft_uniform)
    dd = _dev(drafts)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ids, vb = vpa.top_tokens(x, v, wd, s, 8192, stream=side)
    st = vpa.block_stats(x, v, wd, s, 8192, stream=side)
    ids2, _ = vpa.combine_stats(st, stream=side)
    dst, bst = vpa.verify_stats(x, v, wd, s, r, k, stream=side)
    out = vpa.greedy_verify(dst, bst, dd, stream=side)
    side.synchronize()
    assert torch.equal(ids.cpu(), tgt) and torch.equal(ids2.cpu(), tgt)
    assert torch.equal(vb.cpu().to(torch.int64) & 0xFFFFFFFF, vals)
    for a, b in zip(out, oracle.greedy_verify_logits(w.logits, v, drafts)):
        assert torch.equal(a.cpu(), b)


def test_side_stream_temporaries_are_not_handed_out_early():
    """Temporaries a call frees before its kernels have run (top_tokens'
    workspace, verify_ragged's row lists and statistics) come from the given
    stream's pool: a same-size allocation filled on the default stream while
    the side stream is still busy cannot overwrite them."""
    w = workloads.config3()
    v, wd, s, r, k = w.vocab, w.shard_width, w.n_shards, w.n_req, w.k
    x = _dev(w.logits)
    n = x.shape[0]
    tgt, vals = oracle.argmax(w.logits, v)
    cu = torch.arange(0, (r + 1) * k, k, dtype=torch.int32)
    drafts = workloads.compose_drafts(tgt.reshape(r, k + 1), w.draft_plan, w.draft_uniform)
    want = oracle.greedy_verify_ragged(w.logits, v, cu, drafts.reshape(-1))
    busy = torch.empty(1 << 28, dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _ in range(16):                      # keeps the side stream busy for about 1 ms
            busy.fill_(1)
    # the caller's own inputs stay referenced until the side stream is done
    cu_d, drafts_d = _dev(cu), _dev(drafts.reshape(-1))
    torch.cuda.synchronize()
    ids, vb = vpa.top_tokens(x, v, wd, s, 8192, stream=side)
    out = vpa.verify_ragged(x, v, wd, s, cu_d, drafts_d, r * k, stream=side)
    # the sizes of every temporary above, allocated and filled on the default stream
    junk = [torch.empty(max(vpa.top_tokens_workspace(v, wd, s, n, 8192), 8), dtype=torch.uint8,
                        device=DEV),
            torch.empty(r * k + r, dtype=torch.int32, device=DEV),
            torch.empty(s * (r * k * vpa.stats_slots(wd, s, 8192) + r * vpa.stats_slots(wd, s, 1024))
                        * 2, dtype=torch.int32, device=DEV)]
    for t in junk:
        t.fill_(-1)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(ids.cpu(), tgt)
    assert torch.equal(vb.cpu().to(torch.int64) & 0xFFFFFFFF, vals)
    for a, b, nm in zip(out, want, ("out_tokens", "num_sampled", "num_rejected", "target_ids")):
        assert torch.equal(a.cpu(), b), nm


def test_synthetic_counts_must_be_int32_per_request():
    """accept must be a contiguous int32 device tensor with one entry per request."""
    w = workloads.config3()
    x = _dev(w.logits)
    dst, bst = vpa.verify_stats(x, w.vocab, w.shard_width, w.n_shards, w.n_req, w.k)
    drafts = torch.zeros((w.n_req, w.k), dtype=torch.int32, device=DEV)
    for bad in (torch.zeros(w.n_req, dtype=torch.int64, device=DEV),
                torch.zeros(w.n_req + 1, dtype=torch.int32, device=DEV),
                torch.zeros(w.n_req, dtype=torch.int32)):
        with pytest.raises(ValueError):
            vpa.greedy_verify(dst, bst, drafts, accept=bad)


def test_verify_ragged_needs_the_rows_the_requests_own():
    """verify_ragged refuses logits with fewer rows than cu[-1] + R."""
    x = torch.zeros((6, 1000), dtype=torch.bfloat16, device=DEV)
    cu = torch.tensor([0, 2, 5], dtype=torch.int32, device=DEV)     # 5 drafts + 2 bonus rows = 7
    drafts = torch.zeros(5, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="own 7"):
        vpa.verify_ragged(x, 1000, 500, 2, cu, drafts, 5)


def test_stale_runtime_error_is_left_to_its_owner():
    """A failed, unrelated HIP runtime call earlier in the process (here an
    invalid device number, a host-side argument error) neither fails the
    library's next call nor is consumed by it."""
    w = workloads.config2()
    v, wd, s = w.vocab, w.shard_width, w.n_shards
    x = _dev(w.logits)
    n = x.shape[0]
    ws = torch.empty(vpa.top_tokens_workspace(v, wd, s, n, 8192), dtype=torch.uint8, device=DEV)
    ids = torch.empty(n, dtype=torch.int32, device=DEV)
    vals = torch.empty(n, dtype=torch.int32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    hip = ctypes.CDLL("libamdhip64.so")
    assert hip.hipSetDevice(999) != 0
    status = vpa.lib().vpa_top_tokens(ctypes.c_void_p(x.data_ptr()), vpa.VPA_BF16, x.stride(0),
                                      vpa.Vocab(v, wd, s), n, 8192, ctypes.c_void_p(ws.data_ptr()),
                                      ws.numel(), None, ctypes.c_void_p(ids.data_ptr()),
                                      ctypes.c_void_p(vals.data_ptr()), None, stream)
    stale = hip.hipGetLastError()
    assert status == vpa.VPA_OK, vpa.last_error()
    assert stale != 0                     # still there for the code that caused it
    want_ids, want_vals = oracle.argmax(w.logits, v)
    assert_same(ids, want_ids, "ids after a stale error")
    assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_vals, "vals after a stale error")


def test_hip_graph_replays_match_eager():
    """The draft argmax and the verification captured in one HIP graph: every
    replay, with new logits copied in and eager work and synchronisation in
    between, equals the eager calls on the same data (and the oracle)."""
    w = workloads.config3()
    v, wd, s, r, k = w.vocab, w.shard_width, w.n_shards, w.n_req, w.k
    x_static = _dev(w.logits).clone()
    drafts_static = torch.zeros((r, k), dtype=torch.int32, device=DEV)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):                      # warm the allocator off the default stream
        vpa.top_tokens(x_static, v, wd, s, 8192)
        vpa.greedy_verify(*vpa.verify_stats(x_static, v, wd, s, r, k), drafts_static)
    torch.cuda.current_stream().wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_ids, g_vals = vpa.top_tokens(x_static, v, wd, s, 8192)
        dst, bst = vpa.verify_stats(x_static, v, wd, s, r, k)
        g_out = vpa.greedy_verify(dst, bst, drafts_static)
    for rep in range(4):
        g = torch.Generator().manual_seed(600 + rep)
        x_cpu = (torch.randn(w.logits.shape, generator=g) * 3).to(torch.bfloat16)
        tgt, _ = oracle.argmax(x_cpu, v)
        plan = (torch.rand((r, k), generator=g) < 0.6).to(torch.int8)
        drafts = workloads.compose_drafts(tgt.reshape(r, k + 1), plan,
                                          torch.zeros((r, k), dtype=torch.int32))
        x_static.copy_(_dev(x_cpu))
        drafts_static.copy_(_dev(drafts))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e_ids, e_vals = vpa.top_tokens(x_static, v, wd, s, 8192)       # eager, same data
        e_out = vpa.greedy_verify(*vpa.verify_stats(x_static, v, wd, s, r, k), drafts_static)
        torch.cuda.synchronize()
        assert torch.equal(g_ids, e_ids) and torch.equal(g_vals, e_vals), rep
        for a, b in zip(g_out, e_out):
            assert torch.equal(a, b), rep
        want = oracle.greedy_verify_logits(x_cpu, v, drafts)
        for a, b in zip(g_out, want):
            assert_same(a, b, f"graph replay {rep} vs oracle")


def _chunk_case(n, vocab, ld, seed):
    """bf16 rows with planted maxima where the chunked statistics of
    vpa_top_tokens (4096-column chunks) could go wrong; padding columns
    [vocab, ld) hold +inf and NaN, which must never be read."""
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((n, ld), generator=g) * 3).to(torch.bfloat16)
    x[:, vocab:] = float("inf")
    if ld > vocab + 1:
        x[:, vocab + 1] = float("nan")
    big = 1e4
    plants = [
        [(0, big)],                                          # first column
        [(vocab - 1, big)],                                  # last column
        [(4095, big), (4096, big)],                          # tie across a chunk edge
        [(vocab - 1, big), (max(vocab - 4097, 0), big)],     # tie, the lower id in another chunk
        [(min(5000, vocab - 1), None), (vocab - 1, None)],   # NaNs: the first wins
        "neg_inf",                                           # every column -inf
        "signed_zeros",                                      # -0 everywhere, +0 later: keys tie
        [(min(8191, vocab - 1), float("inf")), (min(8192, vocab - 1), float("inf"))],
    ]
    for r, plant in enumerate(plants[:n]):
        if plant == "neg_inf":
            x[r, :vocab] = float("-inf")
        elif plant == "signed_zeros":
            x[r, :vocab] = -0.0
            x[r, min(7000, vocab - 1)] = 0.0
        else:
            for col, val in plant:
                col = min(col, vocab - 1)
                if val is None:   # a NaN with a payload of its own
                    x[r, col] = torch.tensor([0x7FC1 + col % 7], dtype=torch.int16).view(torch.bfloat16)
                else:
                    x[r, col] = val
    return x


@pytest.mark.parametrize("n,vocab,ld", [
    (64, 200064, 200064),           # the argmax workload's vocabulary
    (1024, 200064, 200064),         # its 1024-row batch, the largest chunked one at this width
    (37, 4096 * 3 + 8, 4096 * 3 + 32),  # a short last chunk, padding columns
    (9, 8, 16),                     # one vector per row
    (300, 4096, 4096),              # exactly one chunk per row
    (12, (1 << 24) - 8, (1 << 24) - 8),  # the largest vocabulary, 4096 chunks per row
])
def test_top_tokens_chunked_statistics(n, vocab, ld):
    """Small bf16 batches take their top_tokens statistics from the chunked
    launch.  Its ids and value bits, with and without the epilogue, equal the
    oracle's, and equal the per-block launch's on the same data (a view
    offset by one element is not 16-byte aligned, so it takes that path)."""
    assert vocab % 8 == 0 and ld % 8 == 0 and n * vocab * 2 <= 1024 * 200064 * 2
    x_cpu = _chunk_case(n, vocab, ld, seed=n + vocab)
    want_ids, want_vals = oracle.argmax(x_cpu[:, :vocab].contiguous(), vocab)
    x = _dev(x_cpu)
    s = 2
    w = -(-vocab // s)
    _announce(f"chunked top_tokens {n} x {vocab} (ld {ld})")
    ids, vals = vpa.top_tokens(x, vocab, w, s)
    assert_same(ids, want_ids, "chunked ids")
    assert_same(vals.to(torch.int64) & 0xFFFFFFFF, want_vals, "chunked value bits")
    shifted = torch.empty((n, ld + 8), dtype=torch.bfloat16, device=DEV)
    xv = shifted[:, 1:1 + ld]
    xv.copy_(x)
    assert xv.data_ptr() % 16 != 0
    ids2, vals2 = vpa.top_tokens(xv, vocab, w, s)
    assert_same(ids2, want_ids, "per-block ids on the same data")
    assert_same(vals2.to(torch.int64) & 0xFFFFFFFF, want_vals, "per-block value bits")
    # the epilogue after chunked statistics
    g = torch.Generator().manual_seed(7)
    d2t = torch.randint(0, 1000, (vocab,), generator=g, dtype=torch.int64)
    ids3, vals3, mapped = vpa.top_tokens(x, vocab, w, s, d2t=_dev(d2t), scale=1 / 0.7)
    assert_same(ids3, want_ids, "chunked ids with the epilogue")
    assert_same(mapped, oracle.map_ids(want_ids, d2t), "chunked mapped ids")
    assert_same(vals3.to(torch.int64) & 0xFFFFFFFF,
                oracle.scale_bits(want_vals, 1 / 0.7), "chunked scaled maxima")


def test_empty_batch_gpu():
    x = torch.empty((0, 1000), dtype=torch.bfloat16, device=DEV)
    st = vpa.block_stats(x, 1000, 125, 8, 256)
    assert st.shape == (8, 0, 2, 2)
    ids, vals = vpa.top_tokens(x, 1000, 125, 8, 256)
    assert ids.numel() == 0
    ids, vals = vpa.combine_stats(st)
    assert ids.numel() == 0
    dst, bst = vpa.verify_stats(x, 1000, 125, 8, 0, 3)
    out, ns, nr, tg = vpa.greedy_verify(dst, bst, torch.empty((0, 3), dtype=torch.int32, device=DEV))
    assert out.shape == (0, 4)
    torch.cuda.synchronize()
