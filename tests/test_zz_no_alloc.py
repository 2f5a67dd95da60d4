"""vpa_top_tokens_noalloc, the entry point for callers that cannot allocate,
called through the C ABI: its outputs equal vpa_top_tokens' (and the
oracle's) on two calls in a row, the second with a smaller input, at the
largest size its device array holds, and with the epilogue; one row past
that size is refused before anything is enqueued."""
import ctypes

import pytest
import torch

import oracle
import vocab_argmax_amd as vpa
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _announce(msg):
    print(f"[noalloc] {msg}", flush=True)


def _noalloc(x, vocab, w, s, block, d2t=None, scale=1.0):
    """One call of vpa_top_tokens_noalloc through ctypes; every output is
    allocated here, before the call."""
    n = x.shape[0]
    ids = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    vals = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    mapped = torch.full((n,), -7, dtype=torch.int64, device=DEV) if d2t is not None else None
    epi = None
    if d2t is not None or scale != 1.0:
        epi = ctypes.pointer(vpa.Epilogue(None if d2t is None else d2t.data_ptr(),
                                          0 if d2t is None else d2t.numel(), scale))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = vpa.lib().vpa_top_tokens_noalloc(
        ctypes.c_void_p(x.data_ptr()), vpa.VPA_BF16 if x.dtype == torch.bfloat16 else vpa.VPA_F32,
        x.stride(0), vpa.Vocab(vocab, w, s), n, block, epi, ctypes.c_void_p(ids.data_ptr()),
        ctypes.c_void_p(vals.data_ptr()), None if mapped is None else ctypes.c_void_p(mapped.data_ptr()),
        stream)
    assert st == vpa.VPA_OK, vpa.last_error()
    return ids, vals, mapped


def _same(a, b, what):
    torch.cuda.synchronize()
    assert torch.equal(a.cpu(), b.cpu()), what


def test_noalloc_matches_top_tokens_on_consecutive_calls():
    # first call: the 4096-row workload with the epilogue (D2T table, scale 1/0.7)
    w4 = workloads.config4(device=DEV)
    x4 = w4.logits
    v, wd, s = w4.vocab, w4.shard_width, w4.n_shards
    g = torch.Generator().manual_seed(4004)
    d2t = torch.randint(0, 1000, (v,), generator=g, dtype=torch.int64).to(DEV)
    _announce(f"{w4.name}: noalloc with epilogue")
    got = _noalloc(x4, v, wd, s, 8192, d2t=d2t, scale=1 / 0.7)
    want = vpa.top_tokens(x4, v, wd, s, 8192, d2t=d2t, scale=1 / 0.7)
    for a, b, nm in zip(got, want, ("ids", "val_bits", "mapped")):
        _same(a, b, f"config4 {nm}")
    # second call, smaller: 32 x 151936, 2 shards; the array still holds the
    # first call's statistics, which must not leak into this result
    w2 = workloads.config2()
    x2 = w2.logits.to(DEV)
    _announce(f"{w2.name}: noalloc after a larger call")
    ids, vals, _ = _noalloc(x2, w2.vocab, w2.shard_width, w2.n_shards, 8192)
    want_ids, want_vals = vpa.top_tokens(x2, w2.vocab, w2.shard_width, w2.n_shards, 8192)
    _same(ids, want_ids, "config2 ids")
    _same(vals, want_vals, "config2 val_bits")
    o_ids, o_vals = oracle.argmax(w2.logits, w2.vocab)
    _same(ids, o_ids, "config2 ids vs oracle")
    _same(vals.to(torch.int64) & 0xFFFFFFFF, o_vals, "config2 values vs oracle")


def test_noalloc_at_its_size_limit():
    """V = 1001 over 8 shards of 126 with 256-blocks: 16 statistics (128 B)
    per row (V is not a multiple of 8, so these are the per-block
    statistics), so 32768 rows fill the 4 MiB array exactly; one more row is
    refused with nothing enqueued."""
    v, wd, s, b = 1001, 126, 8, 256
    per_row = vpa.top_tokens_workspace(v, wd, s, 1, b)
    n = vpa.NOALLOC_WORKSPACE_BYTES // per_row
    assert n * per_row == vpa.NOALLOC_WORKSPACE_BYTES and n == 32768
    g = torch.Generator(device=DEV).manual_seed(5)
    x = (torch.randn((n + 1, v), generator=g, device=DEV) * 3).to(torch.bfloat16)
    x[::7, 17] = x[::7, 903] = 64.0                 # planted ties, as in the small workload
    _announce(f"{n} rows x {v}: noalloc at the limit")
    ids, vals, _ = _noalloc(x[:n], v, wd, s, b)
    want_ids, want_vals = vpa.top_tokens(x[:n], v, wd, s, b)
    _same(ids, want_ids, "limit ids")
    _same(vals, want_vals, "limit val_bits")
    rows = torch.arange(0, n, 997)
    o_ids, o_vals = oracle.argmax(x[rows.to(DEV)].cpu(), v)
    _same(ids[rows.to(DEV)], o_ids, "limit ids vs oracle (sampled rows)")
    ids2 = torch.full((n + 1,), -7, dtype=torch.int32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = vpa.lib().vpa_top_tokens_noalloc(ctypes.c_void_p(x.data_ptr()), vpa.VPA_BF16, v,
                                          vpa.Vocab(v, wd, s), n + 1, b, None,
                                          ctypes.c_void_p(ids2.data_ptr()), None, None, stream)
    assert st == vpa.VPA_ERR_INVALID and "VPA_NOALLOC_WORKSPACE_BYTES" in vpa.last_error()
    torch.cuda.synchronize()
    assert bool((ids2 == -7).all())                  # nothing was written


def test_noalloc_binding_and_graph_capture():
    """The binding's top_tokens_noalloc, with caller-supplied outputs, captured
    in a HIP graph and replayed with new logits: every replay equals the
    eager vpa_top_tokens call on the same data."""
    w = workloads.config3()
    v, wd, s = w.vocab, w.shard_width, w.n_shards
    x = w.logits.to(DEV).clone()
    n = x.shape[0]
    ids = torch.empty(n, dtype=torch.int32, device=DEV)
    vals = torch.empty(n, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        vpa.top_tokens_noalloc(x, v, wd, s, 8192, ids=ids, val_bits=vals)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vpa.top_tokens_noalloc(x, v, wd, s, 8192, ids=ids, val_bits=vals)
    for rep in range(3):
        g = torch.Generator().manual_seed(700 + rep)
        x.copy_((torch.randn(x.shape, generator=g) * 3).to(torch.bfloat16).to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e_ids, e_vals = vpa.top_tokens(x, v, wd, s, 8192)
        _same(ids, e_ids, f"replay {rep} ids")
        _same(vals, e_vals, f"replay {rep} val_bits")
