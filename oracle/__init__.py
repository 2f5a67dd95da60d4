"""CPU oracle for the vocab-parallel greedy argmax -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never calls it and shares no code with
it.  The arithmetic lives in ``vpa_ref.c`` (plain single-threaded C); this
module only marshals CPU tensors into it.

Inputs are CPU ``torch`` tensors: logits of dtype float32 or bfloat16, shape
[rows, ld] with unit column stride, int32 index tensors.  A statistic is a
pair of int32 words: word 0 holds the fp32 bit pattern of the value (read it
as unsigned), word 1 the global token id; statistics tensors have shape
[shards][rows][M][2].  Value bits returned on their own are int64 tensors in
[0, 2^32).
"""
import ctypes
import os

import torch

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libvpa_ref.so")

F32, BF16 = 0, 1
SENTINEL_BITS = 0xFF800000
SENTINEL_ID = 0x7FFFFFFF


def _bind(lib):
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.vpa_ref_stats_slots.argtypes = [i64, i32, i32]
    lib.vpa_ref_stats_slots.restype = i32
    lib.vpa_ref_argmax.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp]
    lib.vpa_ref_argmax.restype = None
    lib.vpa_ref_block_stats.argtypes = [vp, ctypes.c_int, i64, i64, i64, i32, i32, i32, vp, i64,
                                        i32, i32, vp]
    lib.vpa_ref_block_stats.restype = None
    lib.vpa_ref_combine.argtypes = [vp, i32, i64, i32, vp, vp]
    lib.vpa_ref_combine.restype = None
    lib.vpa_ref_greedy_verify.argtypes = [vp, i32, vp, i32, i32, i64, i32, vp, vp, vp, vp, vp, vp]
    lib.vpa_ref_greedy_verify.restype = None
    lib.vpa_ref_greedy_verify_logits.argtypes = [vp, ctypes.c_int, i64, i64, i64, i32, vp, vp,
                                                 vp, vp, vp, vp]
    lib.vpa_ref_greedy_verify_logits.restype = None
    lib.vpa_ref_greedy_verify_ragged.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp, vp,
                                                 vp, vp, vp, vp]
    lib.vpa_ref_greedy_verify_ragged.restype = None
    lib.vpa_ref_greedy_verify_ragged_stats.argtypes = [vp, i32, vp, i32, i32, i64, vp, vp, vp, vp,
                                                       vp, vp, vp, vp]
    lib.vpa_ref_greedy_verify_ragged_stats.restype = None
    lib.vpa_ref_map_ids.argtypes = [vp, i64, vp, i64, vp]
    lib.vpa_ref_map_ids.restype = None
    lib.vpa_ref_scale_bits.argtypes = [ctypes.c_uint32, ctypes.c_float]
    lib.vpa_ref_scale_bits.restype = ctypes.c_uint32
    return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"oracle handles float32 and bfloat16 logits, not {t.dtype}")


def _check_logits(x: torch.Tensor) -> int:
    if x.device.type != "cpu":
        raise ValueError("oracle runs on CPU tensors")
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("logits must be 2-D with unit column stride")
    return x.stride(0) if x.shape[0] > 1 else x.shape[1]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None


def _flags(flags, n):
    """Optional per-request flags as a contiguous uint8 [n] tensor (None stays None)."""
    if flags is None:
        return None
    flags = torch.as_tensor(flags).to("cpu").ne(0).to(torch.uint8).contiguous()
    if flags.numel() != n:
        raise ValueError(f"{flags.numel()} flags for {n} requests")
    return flags


def _counts(accept, n):
    """Optional synthetic accept counts as a contiguous int32 [n] tensor (None stays None)."""
    if accept is None:
        return None
    accept = torch.as_tensor(accept).to("cpu").to(torch.int32).reshape(-1).contiguous()
    if accept.numel() != n:
        raise ValueError(f"{accept.numel()} accept counts for {n} requests")
    return accept


class Oracle:
    """Marshalling over one build of vpa_ref.c (the default build, or a test's
    deliberately broken copy used to show that the pins catch mistakes)."""

    def __init__(self, lib_path: str):
        self.lib = _bind(ctypes.CDLL(lib_path))

    def stats_slots(self, shard_width: int, n_shards: int, block: int) -> int:
        """Slots per shard (M): the most global blocks any shard touches."""
        return int(self.lib.vpa_ref_stats_slots(shard_width, n_shards, block))

    def argmax(self, x: torch.Tensor, vocab: int):
        """Full-row argmax over columns [0, vocab): (ids int32[N], val_bits int64[N])."""
        ld = _check_logits(x)
        n = x.shape[0]
        ids = torch.empty(n, dtype=torch.int32)
        vals = torch.empty(n, dtype=torch.int32)
        if n:
            self.lib.vpa_ref_argmax(_ptr(x), _dtype_code(x), ld, n, vocab, _ptr(ids), _ptr(vals))
        return ids, vals.to(torch.int64) & 0xFFFFFFFF

    def block_stats(self, x: torch.Tensor, vocab: int, shard_width: int, n_shards: int,
                    block: int, rows: torch.Tensor = None, first_shard: int = 0,
                    n_local: int = None):
        """Per-block (value bits, id) statistics, layout [n_local][n_rows][M][2] int32."""
        ld = _check_logits(x)
        if n_local is None:
            n_local = n_shards - first_shard
        n_rows = x.shape[0] if rows is None else rows.numel()
        m = self.stats_slots(shard_width, n_shards, block)
        out = torch.empty((n_local, n_rows, m, 2), dtype=torch.int32)
        if rows is not None:
            rows = rows.to(torch.int32).contiguous()
        if n_rows:
            self.lib.vpa_ref_block_stats(_ptr(x), _dtype_code(x), ld, vocab, shard_width,
                                         n_shards, first_shard, n_local, _ptr(rows), n_rows,
                                         block, m, _ptr(out))
        return out

    def combine(self, stats: torch.Tensor):
        """Rank-order combine of [S][N][M][2] statistics -> (ids int32[N], val_bits int64[N])."""
        stats = stats.contiguous()
        s, n, m, _ = stats.shape
        ids = torch.empty(n, dtype=torch.int32)
        vals = torch.empty(n, dtype=torch.int32)
        if n:
            self.lib.vpa_ref_combine(_ptr(stats), s, n, m, _ptr(ids), _ptr(vals))
        return ids, vals.to(torch.int64) & 0xFFFFFFFF

    def greedy_verify(self, draft_stats: torch.Tensor, bonus_stats: torch.Tensor,
                      draft_ids: torch.Tensor, accept=None):
        """Greedy verification from gathered statistics.

        draft_stats [S][R*K][Md][2], bonus_stats [S][R][Mb][2], draft_ids int32 [R][K];
        accept: optional synthetic accept counts [R] (>= 0: accept that many
        drafts whatever they are; < 0: real acceptance).
        Returns (out_tokens [R][K+1], num_sampled [R], num_rejected [R], target_ids [R][K+1]).
        """
        draft_stats = draft_stats.contiguous()
        bonus_stats = bonus_stats.contiguous()
        draft_ids = draft_ids.to(torch.int32).contiguous()
        r, k = draft_ids.shape
        s, _, md, _ = draft_stats.shape
        mb = bonus_stats.shape[2]
        acc = _counts(accept, r)
        out, ns, nr, tg = _verify_outputs(r, k)
        if r:
            self.lib.vpa_ref_greedy_verify(_ptr(draft_stats), md, _ptr(bonus_stats), mb, s, r, k,
                                           _ptr(draft_ids), _ptr(acc), _ptr(out), _ptr(ns),
                                           _ptr(nr), _ptr(tg))
        return out, ns, nr, tg

    def greedy_verify_logits(self, x: torch.Tensor, vocab: int, draft_ids: torch.Tensor,
                             accept=None):
        """Greedy verification from full logits: request r owns rows r*(K+1)..r*(K+1)+K;
        accept: optional synthetic accept counts [R]."""
        ld = _check_logits(x)
        draft_ids = draft_ids.to(torch.int32).contiguous()
        r, k = draft_ids.shape
        if x.shape[0] < r * (k + 1):
            raise ValueError("logits have fewer rows than requests*(K+1)")
        acc = _counts(accept, r)
        out, ns, nr, tg = _verify_outputs(r, k)
        if r:
            self.lib.vpa_ref_greedy_verify_logits(_ptr(x), _dtype_code(x), ld, vocab, r, k,
                                                  _ptr(draft_ids), _ptr(acc), _ptr(out), _ptr(ns),
                                                  _ptr(nr), _ptr(tg))
        return out, ns, nr, tg


    def greedy_verify_ragged(self, x: torch.Tensor, vocab: int, cu: torch.Tensor,
                             draft_ids: torch.Tensor, prefilling=None, accept=None):
        """Ragged greedy verification from full logits.  cu int32 [R+1] cumulative
        draft counts; request r owns rows cu[r]+r..cu[r]+r+K_r; prefilling: optional
        [R] flags (nonzero = still prefilling: samples nothing); accept: optional
        synthetic accept counts [R] (< 0: real acceptance).  Returns
        (out_tokens [cu[R]+R], num_sampled [R], num_rejected [R], target_ids [cu[R]+R])."""
        ld = _check_logits(x)
        cu = cu.to(torch.int32).contiguous()
        draft_ids = draft_ids.to(torch.int32).contiguous()
        r = cu.numel() - 1
        pf = _flags(prefilling, r)
        acc = _counts(accept, r)
        total = int(cu[-1]) if r > 0 else 0
        if x.shape[0] < total + r:
            raise ValueError("logits have fewer rows than drafts + requests")
        out = torch.empty(total + r, dtype=torch.int32)
        ns = torch.empty(r, dtype=torch.int32)
        nr = torch.empty(r, dtype=torch.int32)
        tg = torch.empty(total + r, dtype=torch.int32)
        if r:
            self.lib.vpa_ref_greedy_verify_ragged(_ptr(x), _dtype_code(x), ld, vocab, r, _ptr(cu),
                                                  _ptr(draft_ids), _ptr(pf), _ptr(acc), _ptr(out),
                                                  _ptr(ns), _ptr(nr), _ptr(tg))
        return out, ns, nr, tg

    def greedy_verify_ragged_stats(self, draft_stats: torch.Tensor, bonus_stats: torch.Tensor,
                                   cu: torch.Tensor, draft_ids: torch.Tensor, prefilling=None,
                                   accept=None):
        """Ragged greedy verification from statistics [S][cu[R]][Md][2], [S][R][Mb][2]."""
        draft_stats = draft_stats.contiguous()
        bonus_stats = bonus_stats.contiguous()
        cu = cu.to(torch.int32).contiguous()
        draft_ids = draft_ids.to(torch.int32).contiguous()
        r = cu.numel() - 1
        pf = _flags(prefilling, r)
        acc = _counts(accept, r)
        total = int(cu[-1]) if r > 0 else 0
        s, md, mb = draft_stats.shape[0], draft_stats.shape[2], bonus_stats.shape[2]
        out = torch.empty(total + r, dtype=torch.int32)
        ns = torch.empty(r, dtype=torch.int32)
        nr = torch.empty(r, dtype=torch.int32)
        tg = torch.empty(total + r, dtype=torch.int32)
        if r:
            self.lib.vpa_ref_greedy_verify_ragged_stats(_ptr(draft_stats), md, _ptr(bonus_stats),
                                                        mb, s, r, _ptr(cu), _ptr(draft_ids),
                                                        _ptr(pf), _ptr(acc), _ptr(out), _ptr(ns),
                                                        _ptr(nr), _ptr(tg))
        return out, ns, nr, tg

    def map_ids(self, ids: torch.Tensor, d2t: torch.Tensor):
        """Draft-to-target ids: ids[i] + d2t[ids[i]] (int64), -1 for ids outside d2t."""
        ids = ids.to(torch.int32).contiguous()
        d2t = d2t.to(torch.int64).contiguous()
        out = torch.empty(ids.numel(), dtype=torch.int64)
        if ids.numel():
            self.lib.vpa_ref_map_ids(_ptr(ids), ids.numel(), _ptr(d2t), d2t.numel(), _ptr(out))
        return out

    def scale_bits(self, val_bits: torch.Tensor, scale: float):
        """Reported maxima under a positive scale (int64 tensor of fp32 bits in, same out)."""
        return torch.tensor([self.lib.vpa_ref_scale_bits(int(b) & 0xFFFFFFFF, scale)
                             for b in val_bits.tolist()], dtype=torch.int64)


def _verify_outputs(r, k):
    return (torch.empty((r, k + 1), dtype=torch.int32), torch.empty(r, dtype=torch.int32),
            torch.empty(r, dtype=torch.int32), torch.empty((r, k + 1), dtype=torch.int32))


def ragged_rows(cu: torch.Tensor):
    """Row lists of a ragged verification batch: draft rows cu[r]+r+j (j < K_r)
    back to back, and bonus rows cu[r+1]+r."""
    cu = cu.to(torch.int64)
    r = cu.numel() - 1
    counts = cu[1:] - cu[:-1]
    req = torch.repeat_interleave(torch.arange(r), counts)
    draft = (torch.arange(int(cu[-1])) + req).to(torch.int32)
    bonus = (cu[1:] + torch.arange(r)).to(torch.int32)
    return draft, bonus


def verify_rows(n_req: int, k: int):
    """Row lists of a verification batch: draft rows r*(K+1)+j (j<K) and bonus rows r*(K+1)+K."""
    r = torch.arange(n_req, dtype=torch.int64)
    j = torch.arange(k, dtype=torch.int64)
    draft = (r[:, None] * (k + 1) + j[None, :]).reshape(-1).to(torch.int32)
    bonus = (r * (k + 1) + k).to(torch.int32)
    return draft, bonus


_default = None


def default() -> Oracle:
    """The oracle built from oracle/vpa_ref.c (rebuilt when the source is newer)."""
    global _default
    if _default is None:
        src = os.path.join(_HERE, "vpa_ref.c")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
            _build.build()
        _default = Oracle(_LIB_PATH)
    return _default


def stats_slots(*a, **kw):
    return default().stats_slots(*a, **kw)


def argmax(*a, **kw):
    return default().argmax(*a, **kw)


def block_stats(*a, **kw):
    return default().block_stats(*a, **kw)


def combine(*a, **kw):
    return default().combine(*a, **kw)


def greedy_verify(*a, **kw):
    return default().greedy_verify(*a, **kw)


def greedy_verify_logits(*a, **kw):
    return default().greedy_verify_logits(*a, **kw)


def map_ids(*a, **kw):
    return default().map_ids(*a, **kw)


def scale_bits(*a, **kw):
    return default().scale_bits(*a, **kw)


def greedy_verify_ragged(*a, **kw):
    return default().greedy_verify_ragged(*a, **kw)


def greedy_verify_ragged_stats(*a, **kw):
    return default().greedy_verify_ragged_stats(*a, **kw)
