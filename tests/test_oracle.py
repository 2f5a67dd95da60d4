"""The oracle checked against the pins (CPU only)."""
import pytest
import torch

import oracle
import oracle_pins
import workloads


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)


def test_planted_tie_config1(o):
    """4 x 1000 fp32, ties planted at ids 17 and 903 in rows 1 and 3: the lower id wins."""
    w = workloads.config1()
    ids, vals = o.argmax(w.logits, w.vocab)
    assert ids[1] == 17 and ids[3] == 17
    assert int(vals[1]) == 0x42800000 == int(vals[3])          # 64.0
    st = o.block_stats(w.logits, w.vocab, w.shard_width, w.n_shards, 256)
    assert torch.equal(o.combine(st)[0], ids)


@pytest.mark.parametrize("case", workloads.edge_cases(), ids=lambda c: c.name)
def test_edge_rows(o, case):
    """The planted rows give the answers their construction fixes."""
    x, v, w, s = case.logits, case.vocab, case.shard_width, case.n_shards
    ids, vals = o.argmax(x, v)
    names = case.notes["row_names"]
    row = {n: i for i, n in enumerate(names)}
    assert ids[row["all_-inf_nan_padding"]] == 0 and int(vals[row["all_-inf_nan_padding"]]) == 0xFF800000
    assert ids[row["all_-inf_inf_padding"]] == 0
    assert int(vals[row["nan_only_at_last_valid"]]) == 0x7FC00000
    assert ids[row["nan_only_at_last_valid"]] == v - 1
    assert ids[row["tie_across_edge_0_1"]] == w - 1
    assert ids[row["max_at_id_0"]] == 0
    assert ids[row["max_at_last_valid"]] == v - 1
    assert int(vals[row["neg_zero_pos_zero_max"]]) == 0x80000000
    assert int(vals[row["pos_inf_twice"]]) == 0x7F800000
    assert int(vals[row["neg_nan_before_pos_nan"]]) == (0xFFC12300 if x.dtype == torch.float32 else 0xFFC10000)
    assert bool((ids < v).all())
    # every block size gives the same ids through the statistics
    for b in case.blocks:
        st = o.block_stats(x, v, w, s, b)
        got_ids, got_vals = o.combine(st)
        assert torch.equal(got_ids, ids) and torch.equal(got_vals, vals), b


def test_empty_batch(o):
    x = torch.empty((0, 1000), dtype=torch.float32)
    ids, vals = o.argmax(x, 1000)
    assert ids.numel() == 0
    st = o.block_stats(x, 1000, 125, 8, 256)
    assert st.shape == (8, 0, 2, 2)


def test_verify_invariants_config3(o):
    """Invariants of greedy verification on the 24 x (3+1) batch."""
    w = workloads.config3()
    x, v = w.logits, w.vocab
    tgt_ids, _ = o.argmax(x, v)
    drafts = workloads.compose_drafts(tgt_ids.reshape(w.n_req, w.k + 1), w.draft_plan, w.draft_uniform)
    out, ns, nr, tg = o.greedy_verify_logits(x, v, drafts)
    assert torch.equal(tg.reshape(-1), tgt_ids)
    assert bool(((ns + nr) == w.k + 1).all())
    for r in range(w.n_req):
        n = int(ns[r]) - 1
        assert out[r, :n].tolist() == drafts[r, :n].tolist()
        assert int(out[r, n]) == int(tg[r, n])
        assert bool((out[r, n + 1:] == -1).all())
    # via the statistics at the page's block sizes: 8192 (drafts), 1024 (bonus)
    draft_rows, bonus_rows = oracle.verify_rows(w.n_req, w.k)
    dst = o.block_stats(x, v, w.shard_width, w.n_shards, 8192, rows=draft_rows)
    bst = o.block_stats(x, v, w.shard_width, w.n_shards, 1024, rows=bonus_rows)
    got = o.greedy_verify(dst, bst, drafts)
    for a, b in zip(got, (out, ns, nr, tg)):
        assert torch.equal(a, b)
