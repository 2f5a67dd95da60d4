"""vocab_argmax_amd -- vocab-parallel greedy argmax and greedy verification on
MI355X (gfx950).

A thin binding over libvpa.so, whose C ABI is include/vpa.h.  ctypes loads
the library; the launch entry points are called through _vpa_call, a small
CPython module (csrc/pycall.c) bound to that same loaded library, which
converts Python ints to C arguments at a fraction of ctypes' per-call cost.
This module only marshals arguments: it checks devices, dtypes and strides,
passes ``data_ptr()`` and the current HIP stream, and allocates outputs with
torch.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  If libvpa.so is missing, every call raises.

Statistics tensors are int32 of shape [shards][rows][M][2]: word 0 holds the
fp32 bit pattern of the block maximum, word 1 its global token id (the
library's ``vpa_stat``).  Value bits come back as int32 tensors holding fp32
bit patterns; ``.view(torch.float32)`` reads them as values.

Sources: vLLM PR #34049, "Solution" (per-shard argmax, exchange of
(max value, global index) pairs, reduction over ranks) and vLLM PR #62604,
"Purpose" items 1 and 2 (per-block statistics with global block boundaries,
fused get_top_tokens, greedy verification) and "Test Plan" (rank-order
layout of the statistics).
"""
import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvpa.so")

VPA_OK, VPA_ERR_INVALID, VPA_ERR_UNSUPPORTED, VPA_ERR_HIP = 0, 1, 2, 3
VPA_F32, VPA_BF16 = 0, 1
EMPTY_BITS = 0xFF800000
EMPTY_ID = 0x7FFFFFFF
DRAFT_BLOCK = 8192   # global block size for draft positions (PR #62604, "Purpose" item 1)
BONUS_BLOCK = 1024   # global block size for the bonus position

# Every symbol include/vpa.h declares.
SYMBOLS = ("vpa_stats_slots", "vpa_block_stats", "vpa_verify_stats", "vpa_verify_stats_rows",
           "vpa_ragged_rows", "vpa_combine_stats", "vpa_top_tokens_workspace", "vpa_top_tokens",
           "vpa_top_tokens_noalloc", "vpa_greedy_verify", "vpa_greedy_verify_ragged",
           "vpa_last_error")
NOALLOC_WORKSPACE_BYTES = 4 << 20   # VPA_NOALLOC_WORKSPACE_BYTES


class VpaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"vpa status {status}: {message}")
        self.status = status


class Vocab(ctypes.Structure):
    """vpa_vocab: V valid columns, S shards of W columns."""
    _fields_ = [("vocab", ctypes.c_int64), ("shard_width", ctypes.c_int64),
                ("n_shards", ctypes.c_int32)]


class Epilogue(ctypes.Structure):
    """vpa_epilogue: optional draft-to-target table and positive logit scale."""
    _fields_ = [("d2t", ctypes.c_void_p), ("d2t_len", ctypes.c_int64), ("scale", ctypes.c_float)]


_lib = None
_call_mod = None


def _bind(lib):
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    st = ctypes.c_int
    lib.vpa_stats_slots.argtypes = [i64, i32, i32]
    lib.vpa_stats_slots.restype = i32
    lib.vpa_block_stats.argtypes = [vp, ctypes.c_int, i64, Vocab, i32, i32, vp, i64, i64, i32, vp, vp]
    lib.vpa_block_stats.restype = st
    lib.vpa_verify_stats.argtypes = [vp, ctypes.c_int, i64, Vocab, i32, i32, i64, i32, i32, i32,
                                     vp, vp, vp]
    lib.vpa_verify_stats.restype = st
    ep = ctypes.POINTER(Epilogue)
    lib.vpa_combine_stats.argtypes = [vp, i32, i64, i32, ep, vp, vp, vp, vp]
    lib.vpa_combine_stats.restype = st
    lib.vpa_top_tokens_workspace.argtypes = [Vocab, i64, i32]
    lib.vpa_top_tokens_workspace.restype = sz
    lib.vpa_top_tokens.argtypes = [vp, ctypes.c_int, i64, Vocab, i64, i32, vp, sz, ep, vp, vp, vp,
                                   vp]
    lib.vpa_top_tokens.restype = st
    lib.vpa_top_tokens_noalloc.argtypes = [vp, ctypes.c_int, i64, Vocab, i64, i32, ep, vp, vp, vp,
                                           vp]
    lib.vpa_top_tokens_noalloc.restype = st
    lib.vpa_greedy_verify.argtypes = [vp, i32, vp, i32, i32, i64, i32, vp, vp, vp, vp, vp, vp,
                                      vp]
    lib.vpa_greedy_verify.restype = st
    lib.vpa_verify_stats_rows.argtypes = [vp, ctypes.c_int, i64, Vocab, i32, i32, vp, i64, vp, i64,
                                          i64, i32, i32, vp, vp, vp]
    lib.vpa_verify_stats_rows.restype = st
    lib.vpa_ragged_rows.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.vpa_ragged_rows.restype = st
    lib.vpa_greedy_verify_ragged.argtypes = [vp, i32, vp, i32, i32, i64, vp, i64, vp, vp, vp, vp,
                                             vp, vp, vp, vp]
    lib.vpa_greedy_verify_ragged.restype = st
    lib.vpa_last_error.argtypes = []
    lib.vpa_last_error.restype = ctypes.c_char_p
    return lib


def lib():
    """The loaded libvpa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m vocab_argmax_amd._build` (hipcc, gfx950)")
        loaded = _bind(ctypes.CDLL(LIB_PATH))
        _bind_call(loaded)
        # sizes cached from a previously loaded library do not carry over
        stats_slots.cache_clear()
        top_tokens_workspace.cache_clear()
        _vocab.cache_clear()
        _lib = loaded
    return _lib


def _bind_call(loaded):
    """Point _vpa_call's entry points at the library just loaded."""
    global _call_mod
    try:
        from . import _vpa_call
    except ImportError as e:
        raise RuntimeError("vocab_argmax_amd/_vpa_call is missing: build it with "
                           f"`python -m vocab_argmax_amd._build` ({e})") from None
    for name in _vpa_call.entries():
        _vpa_call.bind(name, ctypes.cast(getattr(loaded, name), ctypes.c_void_p).value)
    _call_mod = _vpa_call


def call():
    """The launch entry points (vpa_block_stats ... vpa_greedy_verify_ragged),
    bound to the loaded libvpa.so: each takes its C arguments in order, a
    vpa_vocab as three ints and an epilogue as None or (d2t, d2t_len, scale),
    and returns the vpa_status."""
    if _lib is None:
        lib()
    return _call_mod


def last_error() -> str:
    return lib().vpa_last_error().decode()


def _check(status):
    if status != VPA_OK:
        raise VpaError(status, last_error())


def _vp(t):
    return None if t is None else t.data_ptr()


def _raw_stream(device):
    """Handle of `device`'s current HIP stream, as an integer."""
    return torch._C._cuda_getCurrentRawStream(device.index if device.index is not None
                                              else torch.cuda.current_device())


def _stream(stream, device):
    """The HIP stream to enqueue on: the given torch stream, else the current
    stream of `device` (the device the call's tensors live on)."""
    if stream is None:
        return _raw_stream(device)
    if stream.device != device:
        raise ValueError(f"stream belongs to {stream.device}, the tensors to {device}")
    return stream.cuda_stream


def _stream_arg(fn):
    """Run `fn` with its `stream` argument, when one is given, as the current
    stream.  Every tensor the call allocates (outputs, the top_tokens workspace,
    the row lists and statistics of verify_ragged) then comes from that
    stream's pool, and the caching allocator hands a freed temporary's memory
    only to later work on the same stream, which runs after the kernels that
    used it."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kwargs)
    return call


def _on(device, fn, *args):
    """Call the library with `device` current (launches go to the current
    device), switching only when another device is current.  The caller's
    tensors live on `device`, so the runtime is initialised and the current
    device can be read without torch.cuda's initialisation check."""
    if device.index is not None and torch._C._cuda_getDevice() != device.index:
        with torch.cuda.device(device):
            return fn(*args)
    return fn(*args)


def _same_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _dtype_code(x):
    if x.dtype == torch.bfloat16:
        return VPA_BF16
    if x.dtype == torch.float32:
        return VPA_F32
    raise TypeError(f"logits must be bfloat16 or float32, not {x.dtype}")


def _logits_ld(x):
    if not x.is_cuda:
        raise ValueError("logits must be a device tensor")
    if x.dim() != 2:
        raise ValueError("logits must be 2-D [rows, columns]")
    if x.shape[1] > 1 and x.stride(1) != 1:
        raise ValueError("logits columns must be contiguous (stride 1)")
    return x.stride(0) if x.shape[0] > 1 else x.shape[1]


def _int32_dev(t, name, device):
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, logits on {device}")
    return t


def _stats_tensor(t, name):
    if t.dtype != torch.int32 or t.dim() != 4 or t.shape[3] != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 [shards][rows][M][2] tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


def _out_tensor(t, name, dtype, n, device):
    """A caller-supplied output: contiguous, of `dtype`, n elements, on `device`."""
    if t.dtype != dtype or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of {n} elements")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


@functools.lru_cache(maxsize=256)
def stats_slots(shard_width: int, n_shards: int, block: int) -> int:
    """M: statistic slots per shard (the most global blocks a shard touches)."""
    m = lib().vpa_stats_slots(shard_width, n_shards, block)
    if m < 0:
        raise ValueError("invalid shard_width / n_shards / block")
    return m


@functools.lru_cache(maxsize=256)
def _vocab(vocab, shard_width, n_shards):
    return Vocab(vocab, shard_width, n_shards)


@_stream_arg
def block_stats(logits, vocab, shard_width, n_shards, block, rows=None, first_shard=0,
                n_local=None, out=None, *, stream=None):
    """Per-block statistics of shards first_shard..first_shard+n_local-1.

    logits [R, ld]: column 0 is global column first_shard*W.  rows: optional
    int32 device tensor of row indices.  Returns int32 [n_local][n_rows][M][2].
    """
    ld = _logits_ld(logits)
    dev = logits.device
    if n_local is None:
        n_local = n_shards - first_shard
    if rows is not None:
        rows = _int32_dev(rows, "rows", dev)
    n_rows = logits.shape[0] if rows is None else rows.numel()
    m = stats_slots(shard_width, n_shards, block)
    if out is None:
        out = torch.empty((n_local, n_rows, m, 2), dtype=torch.int32, device=dev)
    _stats_tensor(out, "out")
    _same_device(dev, out=out)
    if tuple(out.shape) != (n_local, n_rows, m, 2):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(n_local, n_rows, m, 2)}")
    _check(_on(dev, call().vpa_block_stats, logits.data_ptr(), _dtype_code(logits), ld,
               vocab, shard_width, n_shards, first_shard, n_local, _vp(rows), n_rows,
               logits.shape[0], block, out.data_ptr(), _stream(stream, dev)))
    return out


@_stream_arg
def verify_stats(logits, vocab, shard_width, n_shards, n_req, k, block_draft=DRAFT_BLOCK,
                 block_bonus=BONUS_BLOCK, first_shard=0, n_local=None, out=None, *,
                 stream=None):
    """Draft- and bonus-row statistics of a verification batch in one launch.

    Request r owns rows r*(K+1)..r*(K+1)+K of logits.  Returns
    (draft_stats [n_local][n_req*K][Md][2], bonus_stats [n_local][n_req][Mb][2]);
    `out` may supply that pair preallocated.
    """
    ld = _logits_ld(logits)
    dev = logits.device
    if n_local is None:
        n_local = n_shards - first_shard
    if logits.shape[0] < n_req * (k + 1):
        raise ValueError(f"logits has {logits.shape[0]} rows, need {n_req * (k + 1)}")
    md = stats_slots(shard_width, n_shards, block_draft)
    mb = stats_slots(shard_width, n_shards, block_bonus)
    if out is None:
        # one allocation for both: draft statistics first, then bonus statistics
        nd, nb = n_local * n_req * k * md * 2, n_local * n_req * mb * 2
        buf = torch.empty(nd + nb, dtype=torch.int32, device=dev)
        dst = buf.as_strided((n_local, n_req * k, md, 2), (n_req * k * md * 2, md * 2, 2, 1), 0)
        bst = buf.as_strided((n_local, n_req, mb, 2), (n_req * mb * 2, mb * 2, 2, 1), nd)
    else:
        dst, bst = out
        if (tuple(dst.shape) != (n_local, n_req * k, md, 2)
                or tuple(bst.shape) != (n_local, n_req, mb, 2)):
            raise ValueError("preallocated verification statistics have the wrong shape")
        _stats_tensor(dst, "draft_stats")
        _stats_tensor(bst, "bonus_stats")
        _same_device(dev, draft_stats=dst, bonus_stats=bst)
    _check(_on(dev, call().vpa_verify_stats, logits.data_ptr(), _dtype_code(logits), ld,
               vocab, shard_width, n_shards, first_shard, n_local, n_req, k, block_draft,
               block_bonus, dst.data_ptr(), bst.data_ptr(), _stream(stream, dev)))
    return dst, bst


def _epilogue(d2t, scale, device):
    """The epilogue argument of a launch: None, or (d2t address, d2t_len, scale)."""
    if d2t is None and scale == 1.0:
        return None
    if d2t is not None:
        if d2t.dtype != torch.int64 or not d2t.is_cuda or not d2t.is_contiguous() or d2t.dim() != 1:
            raise ValueError("d2t must be a contiguous 1-D int64 device tensor")
        if d2t.device != device:
            raise ValueError(f"d2t is on {d2t.device}, expected {device}")
    return (None if d2t is None else d2t.data_ptr(), 0 if d2t is None else d2t.numel(),
            float(scale))


@_stream_arg
def combine_stats(stats, d2t=None, scale=1.0, *, stream=None):
    """Rank-order combination of [S][N][M][2] statistics.

    Returns (ids int32[N], val_bits int32[N]), plus mapped int64[N] = k + d2t[k]
    when a draft-to-target table d2t is given.  A positive `scale` leaves the
    ids and scales the reported maxima (fp32, round to nearest)."""
    _stats_tensor(stats, "stats")
    s, n, m, _ = stats.shape
    dev = stats.device
    buf = torch.empty(2 * n, dtype=torch.int32, device=dev)
    ids, vals = buf.as_strided((n,), (1,), 0), buf.as_strided((n,), (1,), n)
    mapped = torch.empty(n, dtype=torch.int64, device=dev) if d2t is not None else None
    epi = _epilogue(d2t, scale, dev)
    _check(_on(dev, call().vpa_combine_stats, stats.data_ptr(), s, n, m, epi, ids.data_ptr(),
               vals.data_ptr(), _vp(mapped), _stream(stream, dev)))
    return (ids, vals) if d2t is None else (ids, vals, mapped)


@functools.lru_cache(maxsize=256)
def top_tokens_workspace(vocab, shard_width, n_shards, n_rows, block=DRAFT_BLOCK) -> int:
    return int(lib().vpa_top_tokens_workspace(_vocab(vocab, shard_width, n_shards), n_rows, block))


@_stream_arg
def top_tokens(logits, vocab, shard_width, n_shards, block=DRAFT_BLOCK, workspace=None,
               ids=None, val_bits=None, d2t=None, scale=1.0, mapped=None, *, stream=None):
    """Fused get_top_tokens over all shards of each row -> (ids int32[N], val_bits int32[N]),
    plus mapped int64[N] = k + d2t[k] when a draft-to-target table is given.

    logits [N, ld] holds the S shards side by side (ld >= vocab).  workspace:
    optional uint8 device tensor of at least top_tokens_workspace() bytes.
    scale: positive logit scale; it leaves the ids and scales the maxima.
    """
    ld = _logits_ld(logits)
    n = logits.shape[0]
    dev = logits.device
    if workspace is None and ids is None and val_bits is None:
        # one int32 allocation: the workspace (rounded up to 256 bytes), then
        # ids, then value bits
        need = (top_tokens_workspace(vocab, shard_width, n_shards, n, block) + 255) // 256 * 64
        buf = torch.empty(need + 2 * n, dtype=torch.int32, device=dev)
        ws_ptr, ws_bytes = buf.data_ptr(), 4 * need
        ids = buf.as_strided((n,), (1,), need)
        val_bits = buf.as_strided((n,), (1,), need + n)
    else:
        if workspace is None:
            need = top_tokens_workspace(vocab, shard_width, n_shards, n, block)
            workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
        elif not workspace.is_contiguous() or workspace.device != dev:
            raise ValueError(f"workspace must be a contiguous tensor on {dev}")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        if ids is None and val_bits is None:
            buf = torch.empty(2 * n, dtype=torch.int32, device=dev)
            ids, val_bits = buf.as_strided((n,), (1,), 0), buf.as_strided((n,), (1,), n)
        else:
            ids = (torch.empty(n, dtype=torch.int32, device=dev) if ids is None
                   else _out_tensor(ids, "ids", torch.int32, n, dev))
            val_bits = (torch.empty(n, dtype=torch.int32, device=dev) if val_bits is None
                        else _out_tensor(val_bits, "val_bits", torch.int32, n, dev))
    if d2t is not None:
        mapped = (torch.empty(n, dtype=torch.int64, device=dev) if mapped is None
                  else _out_tensor(mapped, "mapped", torch.int64, n, dev))
    epi = _epilogue(d2t, scale, dev)
    _check(_on(dev, call().vpa_top_tokens, logits.data_ptr(), _dtype_code(logits), ld, vocab,
               shard_width, n_shards, n, block, ws_ptr, ws_bytes, epi, ids.data_ptr(),
               val_bits.data_ptr(), _vp(mapped if d2t is not None else None),
               _stream(stream, dev)))
    return (ids, val_bits) if d2t is None else (ids, val_bits, mapped)


@_stream_arg
def top_tokens_noalloc(logits, vocab, shard_width, n_shards, block=DRAFT_BLOCK, ids=None,
                       val_bits=None, d2t=None, scale=1.0, mapped=None, *, stream=None):
    """top_tokens with the statistics in the library's own device array
    (vpa_top_tokens_noalloc): the C call allocates nothing, so it can run
    under graph capture or where allocation is forbidden; pass ids,
    val_bits (and mapped) to keep this function from allocating them.  The
    statistics must fit NOALLOC_WORKSPACE_BYTES; calls that overlap on one
    GPU share that array and must not run concurrently."""
    ld = _logits_ld(logits)
    n = logits.shape[0]
    dev = logits.device
    if ids is None and val_bits is None:
        buf = torch.empty(2 * n, dtype=torch.int32, device=dev)
        ids, val_bits = buf.as_strided((n,), (1,), 0), buf.as_strided((n,), (1,), n)
    else:
        ids = (torch.empty(n, dtype=torch.int32, device=dev) if ids is None
               else _out_tensor(ids, "ids", torch.int32, n, dev))
        val_bits = (torch.empty(n, dtype=torch.int32, device=dev) if val_bits is None
                    else _out_tensor(val_bits, "val_bits", torch.int32, n, dev))
    if d2t is not None:
        mapped = (torch.empty(n, dtype=torch.int64, device=dev) if mapped is None
                  else _out_tensor(mapped, "mapped", torch.int64, n, dev))
    epi = _epilogue(d2t, scale, dev)
    _check(_on(dev, call().vpa_top_tokens_noalloc, logits.data_ptr(), _dtype_code(logits), ld,
               vocab, shard_width, n_shards, n, block, epi, ids.data_ptr(),
               val_bits.data_ptr(), _vp(mapped if d2t is not None else None),
               _stream(stream, dev)))
    return (ids, val_bits) if d2t is None else (ids, val_bits, mapped)


def _verify_outputs(r, k, with_targets, dev):
    """out_tokens [r][k+1], num_sampled [r], num_rejected [r] and, if asked for,
    target_ids [r][k+1], as views of one int32 allocation."""
    per = r * (k + 1)
    if with_targets:
        buf = torch.empty(2 * per + 2 * r, dtype=torch.int32, device=dev)
        ns, nr = buf.split_with_sizes((2 * per, r, r))[1:]
        return (buf.as_strided((r, k + 1), (k + 1, 1), 0), ns, nr,
                buf.as_strided((r, k + 1), (k + 1, 1), per))
    buf = torch.empty(per + 2 * r, dtype=torch.int32, device=dev)
    ns, nr = buf.split_with_sizes((per, r, r))[1:]
    return buf.as_strided((r, k + 1), (k + 1, 1), 0), ns, nr, None


@_stream_arg
def greedy_verify(draft_stats, bonus_stats, draft_ids, with_targets=True, out=None,
                  accept=None, *, stream=None):
    """Greedy verification from gathered statistics.

    draft_stats [S][R*K][Md][2], bonus_stats [S][R][Mb][2], draft_ids int32 [R][K].
    accept: optional int32 device tensor [R] of synthetic accept counts (>= 0:
    accept that many drafts whatever they are; < 0: real acceptance).
    Returns (out_tokens [R][K+1], num_sampled [R], num_rejected [R], target_ids [R][K+1] or None);
    `out` may supply those four tensors preallocated (the last may be None).
    """
    _stats_tensor(draft_stats, "draft_stats")
    _stats_tensor(bonus_stats, "bonus_stats")
    dev = draft_stats.device
    _int32_dev(draft_ids, "draft_ids", dev)
    r, k = draft_ids.shape
    s = draft_stats.shape[0]
    if bonus_stats.shape[0] != s or draft_stats.shape[1] != r * k or bonus_stats.shape[1] != r:
        raise ValueError("statistics shapes do not match draft_ids [R][K]")
    _same_device(dev, bonus_stats=bonus_stats)
    accept = _accept_counts(accept, r, dev)
    if out is None:
        out_t, ns, nr, tg = _verify_outputs(r, k, with_targets, dev)
    else:
        out_t, ns, nr, tg = out
        for t, shape in ((out_t, (r, k + 1)), (ns, (r,)), (nr, (r,)), (tg, (r, k + 1))):
            if t is not None and (tuple(t.shape) != shape or t.dtype != torch.int32
                                  or not t.is_contiguous()):
                raise ValueError("preallocated verification outputs have the wrong shape/dtype")
        _same_device(dev, out_tokens=out_t, num_sampled=ns, num_rejected=nr, target_ids=tg)
    _check(_on(dev, call().vpa_greedy_verify, draft_stats.data_ptr(), draft_stats.shape[2],
               bonus_stats.data_ptr(), bonus_stats.shape[2], s, r, k, draft_ids.data_ptr(),
               _vp(accept), out_t.data_ptr(), ns.data_ptr(), nr.data_ptr(), _vp(tg),
               _stream(stream, dev)))
    return out_t, ns, nr, tg


def _total_drafts(cu, total_drafts):
    _int32_dev(cu, "cu", cu.device)
    if cu.dim() != 1 or cu.numel() < 1:
        raise ValueError("cu must be a 1-D int32 tensor of n_req+1 cumulative draft counts")
    # reading cu[-1] synchronises with the device; callers that know the total pass it
    return int(cu[-1]) if total_drafts is None else int(total_drafts)


@_stream_arg
def ragged_rows(cu, total_drafts=None, *, stream=None):
    """Row lists of a ragged verification batch from cumulative draft counts
    cu [R+1]: (draft_rows int32[total_drafts], bonus_rows int32[R])."""
    total = _total_drafts(cu, total_drafts)
    n_req = cu.numel() - 1
    buf = torch.empty(total + n_req, dtype=torch.int32, device=cu.device)
    draft_rows, bonus_rows = buf[:total], buf[total:]
    _check(_on(cu.device, call().vpa_ragged_rows, cu.data_ptr(), n_req, total,
               draft_rows.data_ptr(), bonus_rows.data_ptr(), _stream(stream, cu.device)))
    return draft_rows, bonus_rows


@_stream_arg
def verify_stats_rows(logits, vocab, shard_width, n_shards, draft_rows, bonus_rows,
                      block_draft=DRAFT_BLOCK, block_bonus=BONUS_BLOCK, first_shard=0,
                      n_local=None, *, stream=None):
    """Draft- and bonus-row statistics for two explicit row lists in one launch:
    (draft_stats [n_local][len(draft_rows)][Md][2], bonus_stats [n_local][len(bonus_rows)][Mb][2])."""
    ld = _logits_ld(logits)
    dev = logits.device
    if n_local is None:
        n_local = n_shards - first_shard
    _int32_dev(draft_rows, "draft_rows", dev)
    _int32_dev(bonus_rows, "bonus_rows", dev)
    md = stats_slots(shard_width, n_shards, block_draft)
    mb = stats_slots(shard_width, n_shards, block_bonus)
    nd_rows, nb_rows = draft_rows.numel(), bonus_rows.numel()
    nd = n_local * nd_rows * md * 2
    buf = torch.empty(nd + n_local * nb_rows * mb * 2, dtype=torch.int32, device=dev)
    dst = buf[:nd].view(n_local, nd_rows, md, 2)
    bst = buf[nd:].view(n_local, nb_rows, mb, 2)
    _check(_on(dev, call().vpa_verify_stats_rows, logits.data_ptr(), _dtype_code(logits), ld,
               vocab, shard_width, n_shards, first_shard, n_local, draft_rows.data_ptr(),
               nd_rows, bonus_rows.data_ptr(), nb_rows, logits.shape[0], block_draft, block_bonus,
               dst.data_ptr(), bst.data_ptr(), _stream(stream, dev)))
    return dst, bst


def _prefilling_flags(prefilling, n_req, device):
    """Optional per-request prefilling flags: a bool or uint8 device tensor [R]."""
    if prefilling is None:
        return None
    if prefilling.dtype not in (torch.bool, torch.uint8) or not prefilling.is_contiguous():
        raise ValueError("prefilling must be a contiguous bool or uint8 tensor")
    if prefilling.device != device:
        raise ValueError(f"prefilling is on {prefilling.device}, expected {device}")
    if prefilling.numel() != n_req:
        raise ValueError(f"prefilling has {prefilling.numel()} entries for {n_req} requests")
    return prefilling


def _accept_counts(accept, n_req, device):
    """Optional synthetic accept counts: a contiguous int32 device tensor [R]."""
    if accept is None:
        return None
    _int32_dev(accept, "accept", device)
    if accept.numel() != n_req:
        raise ValueError(f"accept has {accept.numel()} entries for {n_req} requests")
    return accept


@_stream_arg
def greedy_verify_ragged(draft_stats, bonus_stats, cu, draft_ids, total_drafts=None,
                         with_targets=True, prefilling=None, accept=None, *, stream=None):
    """Ragged greedy verification from statistics.  cu int32 [R+1] cumulative
    draft counts; draft_ids int32 [total_drafts]; prefilling: optional bool or
    uint8 [R], true for a request still prefilling, which samples nothing (-1
    in its slots, 0 sampled, 0 rejected); accept: optional int32 [R] synthetic
    accept counts as for greedy_verify, with K_r for K.  Returns (out_tokens [total+R],
    num_sampled [R], num_rejected [R], target_ids [total+R] or None); request
    r's K_r+1 outputs sit at offset cu[r]+r."""
    _stats_tensor(draft_stats, "draft_stats")
    _stats_tensor(bonus_stats, "bonus_stats")
    total = _total_drafts(cu, total_drafts)
    n_req = cu.numel() - 1
    dev = bonus_stats.device
    _same_device(dev, cu=cu, draft_stats=draft_stats)
    _int32_dev(draft_ids, "draft_ids", dev)
    prefilling = _prefilling_flags(prefilling, n_req, dev)
    accept = _accept_counts(accept, n_req, dev)
    if draft_ids.numel() != total or draft_stats.shape[1] != total or bonus_stats.shape[1] != n_req:
        raise ValueError("statistics / draft_ids do not match the offsets")
    if draft_stats.shape[0] != bonus_stats.shape[0]:
        raise ValueError("draft and bonus statistics have different shard counts")
    per = total + n_req
    buf = torch.empty(per * (2 if with_targets else 1) + 2 * n_req, dtype=torch.int32, device=dev)
    out, ns, nr = buf[:per], buf[per:per + n_req], buf[per + n_req:per + 2 * n_req]
    tg = buf[per + 2 * n_req:] if with_targets else None
    _check(_on(dev, call().vpa_greedy_verify_ragged, draft_stats.data_ptr(), draft_stats.shape[2],
               bonus_stats.data_ptr(), bonus_stats.shape[2], bonus_stats.shape[0], n_req,
               cu.data_ptr(), total, draft_ids.data_ptr(), _vp(prefilling), _vp(accept),
               out.data_ptr(), ns.data_ptr(), nr.data_ptr(), _vp(tg), _stream(stream, dev)))
    return out, ns, nr, tg


@_stream_arg
def verify_ragged(logits, vocab, shard_width, n_shards, cu, draft_ids, total_drafts=None,
                  block_draft=DRAFT_BLOCK, block_bonus=BONUS_BLOCK, with_targets=True,
                  prefilling=None, accept=None, *, stream=None):
    """The whole ragged verification on one GPU: row lists, statistics, finish.
    logits must hold the total_drafts + R rows the requests own."""
    total = _total_drafts(cu, total_drafts)
    n_req = cu.numel() - 1
    if logits.shape[0] < total + n_req:
        raise ValueError(f"logits has {logits.shape[0]} rows, the requests own {total + n_req}")
    draft_rows, bonus_rows = ragged_rows(cu, total, stream=stream)
    dst, bst = verify_stats_rows(logits, vocab, shard_width, n_shards, draft_rows, bonus_rows,
                                 block_draft, block_bonus, stream=stream)
    return greedy_verify_ragged(dst, bst, cu, draft_ids, total, with_targets, prefilling, accept,
                                stream=stream)
