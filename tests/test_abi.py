"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects invalid arguments before any HIP call (so these calls
need no GPU; pointers passed here are never dereferenced)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import bruteforce as bf
import vocab_argmax_amd as vpa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "vpa.h")
# aligned, never dereferenced by a rejected call; above 2^32, so that an
# address passed through a 32-bit slot fails loudly
FAKE = ctypes.c_void_p(0x7F0000010000)
FAKE_ODD = ctypes.c_void_p(0x7F0000010001)


def _as_python(arg):
    """One ctypes argument as the _vpa_call module takes it (a list: a vocab
    struct becomes three ints)."""
    if isinstance(arg, ctypes.c_void_p):
        return [arg.value]
    if isinstance(arg, vpa.Vocab):
        return [arg.vocab, arg.shard_width, arg.n_shards]
    if isinstance(arg, ctypes.POINTER(vpa.Epilogue)):
        e = arg.contents
        return [(e.d2t, e.d2t_len, e.scale)]
    return [arg]


class BothPaths:
    """The loaded library, whose launch entry points run twice: through ctypes
    and through the binding's _vpa_call module.  Both must return the same
    status and, on an error, the same message."""

    def __init__(self, loaded):
        self._lib = loaded

    def __getattr__(self, name):
        through_ctypes = getattr(self._lib, name)
        if name not in vpa.call().entries():
            return through_ctypes
        through_module = getattr(vpa.call(), name)

        def both(*args):
            st = through_ctypes(*args)
            msg = vpa.last_error() if st != vpa.VPA_OK else ""
            st2 = through_module(*[a for arg in args for a in _as_python(arg)])
            msg2 = vpa.last_error() if st2 != vpa.VPA_OK else ""
            assert (st2, msg2) == (st, msg), f"{name}: _vpa_call and ctypes disagree"
            return st
        return both


@pytest.fixture(scope="module", params=["ctypes", "ctypes_and_module"])
def lib(request):
    """Every C-ABI test runs on the library through ctypes, then once more
    with each launch also made through the binding's _vpa_call module."""
    return vpa.lib() if request.param == "ctypes" else BothPaths(vpa.lib())


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vpa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(vpa.SYMBOLS), names
    for name in names:
        assert hasattr(lib, name), name


def test_stats_slots_matches_bruteforce(lib):
    for w in (1, 2, 5, 125, 1000, 16753, 25008):
        for s in (1, 2, 3, 8):
            for b in (1, 7, 256, 1024, 8192):
                if w * s > 200000 and b < 64:
                    continue
                want = bf.bf_stats_slots(w, s, b) if w * s <= 20000 else None
                got = lib.vpa_stats_slots(w, s, b)
                if want is not None:
                    assert got == want, (w, s, b)
                assert got >= 1
    assert lib.vpa_stats_slots(0, 1, 1) == -1
    assert lib.vpa_stats_slots(1, 0, 1) == -1
    assert lib.vpa_stats_slots(1, 1, 0) == -1
    # the configurations' slot counts
    assert lib.vpa_stats_slots(76032, 2, 8192) == 10
    assert lib.vpa_stats_slots(50016, 4, 8192) == 7
    assert lib.vpa_stats_slots(50016, 4, 1024) == 50
    assert lib.vpa_stats_slots(25008, 8, 8192) == 4
    assert lib.vpa_stats_slots(25008, 8, 1024) == 26


def V(v, w, s):
    return vpa.Vocab(v, w, s)


def call_block_stats(lib, logits=FAKE, dt=vpa.VPA_BF16, ld=1000, voc=None, first=0, nloc=1,
                     rows=None, n_rows=4, logits_rows=4, block=256, stats=FAKE):
    voc = voc or V(1000, 1000, 1)
    return lib.vpa_block_stats(logits, dt, ld, voc, first, nloc, rows, n_rows, logits_rows, block,
                               stats, None)


@pytest.mark.parametrize("kw,status", [
    (dict(voc=V(0, 1, 1)), vpa.VPA_ERR_INVALID),
    (dict(voc=V(1 << 24, 1 << 24, 1)), vpa.VPA_ERR_INVALID),
    (dict(voc=V(1000, 0, 1)), vpa.VPA_ERR_INVALID),
    (dict(voc=V(1000, 100, 0)), vpa.VPA_ERR_INVALID),
    (dict(voc=V(1000, 100, 9), nloc=1), vpa.VPA_ERR_INVALID),          # 900 < 1000 columns
    (dict(first=-1), vpa.VPA_ERR_INVALID),
    (dict(nloc=0), vpa.VPA_ERR_INVALID),
    (dict(voc=V(1000, 500, 2), first=1, nloc=2), vpa.VPA_ERR_INVALID),
    (dict(ld=999), vpa.VPA_ERR_INVALID),
    (dict(block=0), vpa.VPA_ERR_INVALID),
    (dict(dt=7), vpa.VPA_ERR_UNSUPPORTED),
    (dict(logits=None), vpa.VPA_ERR_INVALID),
    (dict(logits=FAKE_ODD), vpa.VPA_ERR_INVALID),
    (dict(stats=None), vpa.VPA_ERR_INVALID),
    (dict(stats=FAKE_ODD), vpa.VPA_ERR_INVALID),
    (dict(n_rows=-1), vpa.VPA_ERR_INVALID),
    (dict(n_rows=5, logits_rows=4), vpa.VPA_ERR_INVALID),               # identity rows past the buffer
    (dict(voc=V(100, 100, 1), ld=100, block=1, n_rows=1 << 25, logits_rows=1 << 25), vpa.VPA_ERR_INVALID),
])
def test_block_stats_rejects(lib, kw, status):
    assert call_block_stats(lib, **kw) == status
    assert vpa.last_error() != ""


def test_block_stats_ld_covers_only_valid_columns(lib):
    # the last rank of V=1000 over W=334, S=3 holds 332 valid columns; ld=332 is enough,
    # and a zero-row call is a no-op that never touches the pointers
    assert call_block_stats(lib, voc=V(1000, 334, 3), first=2, nloc=1, ld=332, n_rows=0) == vpa.VPA_OK
    assert call_block_stats(lib, voc=V(1000, 334, 3), first=2, nloc=1, ld=331, n_rows=0) == vpa.VPA_ERR_INVALID


def test_empty_batches_are_noops(lib):
    assert call_block_stats(lib, n_rows=0, stats=None) == vpa.VPA_OK
    assert lib.vpa_combine_stats(None, 8, 0, 2, None, None, None, None, None) == vpa.VPA_OK
    assert lib.vpa_top_tokens(FAKE, vpa.VPA_BF16, 1000, V(1000, 125, 8), 0, 256, None, 0, None,
                              None, None, None, None) == vpa.VPA_OK
    assert lib.vpa_verify_stats(FAKE, vpa.VPA_F32, 1000, V(1000, 125, 8), 0, 8, 0, 3, 8192, 1024,
                                None, None, None) == vpa.VPA_OK
    assert lib.vpa_greedy_verify(None, 1, None, 1, 8, 0, 3, None, None, None, None, None, None,
                                 None) == vpa.VPA_OK


def EPI(d2t=None, n=0, scale=1.0):
    return ctypes.pointer(vpa.Epilogue(d2t, n, scale))


def test_combine_rejects(lib):
    cs = lib.vpa_combine_stats
    assert cs(FAKE, 0, 4, 2, None, FAKE, None, None, None) == vpa.VPA_ERR_INVALID
    assert cs(FAKE, 2, 4, 0, None, FAKE, None, None, None) == vpa.VPA_ERR_INVALID
    assert cs(None, 2, 4, 2, None, FAKE, None, None, None) == vpa.VPA_ERR_INVALID
    assert cs(FAKE, 2, 4, 2, None, None, None, None, None) == vpa.VPA_ERR_INVALID
    assert cs(FAKE, 2, 4, 2, None, FAKE, FAKE_ODD, None, None) == vpa.VPA_ERR_INVALID
    assert cs(FAKE, 2, -1, 2, None, FAKE, None, None, None) == vpa.VPA_ERR_INVALID


@pytest.mark.parametrize("epi,mapped", [
    (dict(scale=0.0), None), (dict(scale=-1.0), None), (dict(scale=float("inf")), None),
    (dict(scale=float("nan")), None),
    (dict(d2t=0x10000, n=0), FAKE),            # empty table
    (dict(d2t=0x10004, n=10), FAKE),           # unaligned table
    (dict(d2t=0x10000, n=10), None),           # a table but nowhere to write the mapped ids
    (dict(), FAKE),                             # mapped ids but no table
    (dict(d2t=0x10000, n=10), FAKE_ODD),       # unaligned mapped ids
])
def test_epilogue_rejects(lib, epi, mapped):
    assert lib.vpa_combine_stats(FAKE, 2, 4, 2, EPI(**epi), FAKE, None, mapped, None) == vpa.VPA_ERR_INVALID
    # top_tokens also needs the table to cover the vocabulary
    voc = V(1000, 500, 2)
    assert lib.vpa_top_tokens(FAKE, vpa.VPA_BF16, 1000, voc, 4, 256, FAKE, 1 << 20, EPI(**epi),
                              FAKE, None, mapped, None) == vpa.VPA_ERR_INVALID


def test_top_tokens_d2t_must_cover_vocab(lib):
    voc = V(1000, 500, 2)
    call = lambda n: lib.vpa_top_tokens(FAKE, vpa.VPA_BF16, 1000, voc, 0, 256, FAKE, 1 << 20,
                                        EPI(0x10000, n), FAKE, None, FAKE, None)
    assert call(999) == vpa.VPA_ERR_INVALID
    assert call(1000) == vpa.VPA_OK              # zero rows: validated, nothing enqueued


def test_top_tokens_rejects(lib):
    voc = V(151936, 76032, 2)
    need = lib.vpa_top_tokens_workspace(voc, 32, 8192)
    assert need == 32 * 38 * 8            # 38 chunks of 4096 columns per row (chunk_stats.hip)
    assert lib.vpa_top_tokens_workspace(voc, 0, 8192) == 0
    assert lib.vpa_top_tokens_workspace(voc, 32, 0) == 0
    args = dict(ld=152064, n=32, block=8192, ws=FAKE, wsb=need, ids=FAKE)

    def call(**kw):
        a = {**args, **kw}
        return lib.vpa_top_tokens(FAKE, vpa.VPA_BF16, a["ld"], voc, a["n"], a["block"], a["ws"],
                                  a["wsb"], None, a["ids"], None, None, None)
    assert call(wsb=need - 1) == vpa.VPA_ERR_INVALID
    assert call(ws=None) == vpa.VPA_ERR_INVALID
    assert call(ws=FAKE_ODD) == vpa.VPA_ERR_INVALID
    assert call(ids=None) == vpa.VPA_ERR_INVALID
    assert call(ld=151935) == vpa.VPA_ERR_INVALID
    assert call(block=-3) == vpa.VPA_ERR_INVALID
    assert "workspace" in (call(wsb=1) and vpa.last_error())


def test_verify_rejects(lib):
    voc = V(200064, 50016, 4)
    assert lib.vpa_verify_stats(FAKE, vpa.VPA_BF16, 200064, voc, 0, 4, 24, 0, 8192, 1024, FAKE,
                                FAKE, None) == vpa.VPA_ERR_INVALID
    assert lib.vpa_verify_stats(FAKE, vpa.VPA_BF16, 200064, voc, 0, 4, 24, 3, 0, 1024, FAKE,
                                FAKE, None) == vpa.VPA_ERR_INVALID
    assert lib.vpa_verify_stats(FAKE, vpa.VPA_BF16, 200064, voc, 0, 4, 24, 3, 8192, 1024, None,
                                FAKE, None) == vpa.VPA_ERR_INVALID
    assert lib.vpa_verify_stats(FAKE, vpa.VPA_BF16, 200064, voc, 0, 4, 24, 4097, 8192, 1024, FAKE,
                                FAKE, None) == vpa.VPA_ERR_INVALID
    gv = lib.vpa_greedy_verify
    assert gv(FAKE, 7, FAKE, 50, 4, 24, 4097, FAKE, None, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert gv(FAKE, 7, FAKE, 50, 4, 24, 0, FAKE, None, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert gv(FAKE, 0, FAKE, 50, 4, 24, 3, FAKE, None, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert gv(FAKE, 7, FAKE, 50, 0, 24, 3, FAKE, None, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert gv(FAKE, 7, FAKE, 50, 4, 24, 3, None, None, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert gv(FAKE, 7, FAKE, 50, 4, 24, 3, FAKE, None, FAKE, FAKE, FAKE, FAKE_ODD, None) == vpa.VPA_ERR_INVALID
    assert gv(FAKE, 7, FAKE, 50, 4, -1, 3, FAKE, None, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    # synthetic accept counts must be 4-byte aligned
    assert gv(FAKE, 7, FAKE, 50, 4, 24, 3, FAKE, FAKE_ODD, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID


def test_last_error_is_per_call_message(lib):
    call_block_stats(lib, block=0)
    assert "block" in vpa.last_error()


def test_ragged_rejects(lib):
    voc = V(200064, 50016, 4)
    vsr = lib.vpa_verify_stats_rows
    assert vsr(FAKE, vpa.VPA_BF16, 200064, voc, 0, 4, FAKE, -1, FAKE, 2, 8, 8192, 1024, FAKE,
               FAKE, None) == vpa.VPA_ERR_INVALID
    assert vsr(FAKE, vpa.VPA_BF16, 200064, voc, 0, 4, None, 6, FAKE, 2, 8, 8192, 1024, FAKE,
               FAKE, None) == vpa.VPA_ERR_INVALID
    assert vsr(FAKE, vpa.VPA_BF16, 200064, voc, 0, 4, FAKE, 6, FAKE_ODD, 2, 8, 8192, 1024, FAKE,
               FAKE, None) == vpa.VPA_ERR_INVALID
    assert vsr(FAKE, vpa.VPA_BF16, 200064, voc, 0, 4, FAKE, 6, FAKE, 2, 8, 0, 1024, FAKE,
               FAKE, None) == vpa.VPA_ERR_INVALID
    assert vsr(None, vpa.VPA_BF16, 200064, voc, 0, 4, None, 0, None, 0, 0, 8192, 1024, None,
               None, None) == vpa.VPA_OK                       # nothing to do
    rr = lib.vpa_ragged_rows
    assert rr(FAKE, -1, 0, FAKE, FAKE, None) == vpa.VPA_ERR_INVALID
    assert rr(FAKE, 3, -1, FAKE, FAKE, None) == vpa.VPA_ERR_INVALID
    assert rr(None, 3, 4, FAKE, FAKE, None) == vpa.VPA_ERR_INVALID
    assert rr(FAKE, 3, 4, None, FAKE, None) == vpa.VPA_ERR_INVALID
    assert rr(FAKE_ODD, 3, 4, FAKE, FAKE, None) == vpa.VPA_ERR_INVALID
    assert rr(None, 0, 0, None, None, None) == vpa.VPA_OK
    gr = lib.vpa_greedy_verify_ragged
    assert gr(FAKE, 0, FAKE, 50, 4, 3, FAKE, 6, FAKE, None, None, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert gr(FAKE, 7, FAKE, 50, 4, 3, None, 6, FAKE, None, None, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert gr(FAKE, 7, FAKE, 50, 4, 3, FAKE, 6, None, None, None, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert gr(FAKE, 7, FAKE, 50, 4, 3, FAKE, 6, FAKE, None, None, FAKE, FAKE, FAKE, FAKE_ODD, None) == vpa.VPA_ERR_INVALID
    assert gr(FAKE, 7, FAKE, 50, 4, -2, FAKE, 6, FAKE, None, None, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert gr(FAKE, 7, FAKE, 50, 4, 3, FAKE, 6, FAKE, None, FAKE_ODD, FAKE, FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert gr(None, 7, None, 50, 4, 0, None, 0, None, None, None, None, None, None, None, None) == vpa.VPA_OK


def test_launches_beyond_one_dispatch_are_rejected(lib):
    # A dispatch holds fewer than 2^32 work-items: calls whose statistics fit in
    # 2^31 but whose launch would not are rejected before any HIP call.
    big = (1 << 26) + 1                          # one 64-lane wavefront per row at V=16384
    assert call_block_stats(lib, voc=V(16384, 16384, 1), ld=16384, block=16384, n_rows=big,
                            logits_rows=big) == vpa.VPA_ERR_INVALID
    assert "dispatch" in vpa.last_error()
    assert lib.vpa_combine_stats(FAKE, 1, big, 1, None, FAKE, None, None, None) == vpa.VPA_ERR_INVALID
    assert "dispatch" in vpa.last_error()
    ws = vpa.lib().vpa_top_tokens_workspace(V(16384, 16384, 1), big, 16384)
    assert lib.vpa_top_tokens(FAKE, vpa.VPA_BF16, 16384, V(16384, 16384, 1), big, 16384, FAKE, ws,
                              None, FAKE, None, None, None) == vpa.VPA_ERR_INVALID
    assert "dispatch" in vpa.last_error()
    assert lib.vpa_verify_stats(FAKE, vpa.VPA_BF16, 16384, V(16384, 16384, 1), 0, 1, big // 2 + 1, 1,
                                16384, 16384, FAKE, FAKE, None) == vpa.VPA_ERR_INVALID
    assert "dispatch" in vpa.last_error()
    req = (1 << 22) + 1                          # 16 wavefronts per request at K=15
    assert lib.vpa_greedy_verify(FAKE, 1, FAKE, 1, 1, req, 15, FAKE, None, FAKE, FAKE, FAKE, None,
                                 None) == vpa.VPA_ERR_INVALID
    assert "dispatch" in vpa.last_error()
    req = (1 << 24) + 1                          # one 256-thread workgroup per request
    assert lib.vpa_greedy_verify_ragged(FAKE, 1, FAKE, 1, 1, req, FAKE, 0, None, None, None, FAKE,
                                        FAKE, FAKE, None, None) == vpa.VPA_ERR_INVALID
    assert "dispatch" in vpa.last_error()


def test_header_is_plain_c_and_cxx(tmp_path):
    """include/vpa.h compiles as strict C99 and as C++11, warnings as errors."""
    cc = shutil.which("gcc")
    cxx = shutil.which("g++")
    if not cc or not cxx:
        pytest.skip("gcc/g++ not available")
    src = tmp_path / "h.c"
    src.write_text('#include "vpa.h"\nint main(void) { return 0; }\n')
    inc = os.path.dirname(HEADER)
    for cmd in ([cc, "-std=c99", "-pedantic"], [cxx, "-std=c++11", "-pedantic", "-x", "c++"]):
        subprocess.run(cmd + ["-Wall", "-Wextra", "-Werror", "-I", inc, "-fsyntax-only", str(src)],
                       check=True)


def test_plain_c_program_links_and_calls(tmp_path):
    """A C99 program links against the built library and gets host-side
    answers (slots, workspace, rejections, empty batches) without a GPU."""
    cc = shutil.which("gcc")
    if not cc:
        pytest.skip("gcc not available")
    lib_dir = os.path.dirname(vpa.LIB_PATH)
    exe = tmp_path / "c_consumer"
    here = os.path.dirname(os.path.abspath(__file__))
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.dirname(HEADER),
                    os.path.join(here, "c_consumer.c"), "-L", lib_dir, "-l:libvpa.so",
                    f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "FAIL" not in out.stdout and out.stdout.count("ok ") == 7, out.stdout


def test_sizes_past_the_limits_are_rejected_without_overflow(lib):
    """Shard counts above 2^24 and row counts near 2^63 are rejected at once:
    the host checks never loop over absurd shard counts or overflow."""
    assert lib.vpa_stats_slots(1, (1 << 24) + 1, 1) == -1
    assert lib.vpa_stats_slots(1, 1 << 24, 1 << 30) == 1
    assert call_block_stats(lib, voc=V(1000, 1, (1 << 24) + 1)) == vpa.VPA_ERR_INVALID
    assert "n_shards" in vpa.last_error()
    huge = (1 << 62) + 3
    assert lib.vpa_top_tokens_workspace(V(1000, 1000, 1), huge, 256) == 0
    assert lib.vpa_top_tokens_workspace(V(1000, 1000, 1), 1 << 31, 256) == 0
    assert call_block_stats(lib, n_rows=huge, logits_rows=huge) == vpa.VPA_ERR_INVALID
    assert lib.vpa_top_tokens(FAKE, vpa.VPA_BF16, 1000, V(1000, 125, 8), huge, 256, FAKE, 1 << 40,
                              None, FAKE, None, None, None) == vpa.VPA_ERR_INVALID
    assert lib.vpa_verify_stats(FAKE, vpa.VPA_BF16, 1000, V(1000, 125, 8), 0, 8, huge, 3, 8192,
                                1024, FAKE, FAKE, None) == vpa.VPA_ERR_INVALID


def test_noalloc_top_tokens_rejects_beyond_its_array(lib):
    """vpa_top_tokens_noalloc validates like vpa_top_tokens and refuses, before
    any HIP call, a call whose statistics exceed VPA_NOALLOC_WORKSPACE_BYTES."""
    voc = V(200064, 25008, 8)                    # 32 statistics (256 bytes) per row
    limit = vpa.NOALLOC_WORKSPACE_BYTES
    assert lib.vpa_top_tokens_workspace(voc, 16384, 8192) == limit
    call = lambda n, **kw: lib.vpa_top_tokens_noalloc(
        kw.get("logits", FAKE), vpa.VPA_BF16, kw.get("ld", 200064), voc, n, kw.get("block", 8192),
        None, kw.get("ids", FAKE), None, None, None)
    assert call(16385) == vpa.VPA_ERR_INVALID
    assert "VPA_NOALLOC_WORKSPACE_BYTES" in vpa.last_error()
    assert call(0) == vpa.VPA_OK                 # empty batch: nothing to do
    assert call(4, ids=None) == vpa.VPA_ERR_INVALID
    assert call(4, logits=FAKE_ODD) == vpa.VPA_ERR_INVALID
    assert call(4, ld=200063) == vpa.VPA_ERR_INVALID
    assert call(4, block=0) == vpa.VPA_ERR_INVALID
    assert lib.vpa_top_tokens_noalloc(FAKE, vpa.VPA_BF16, 200064, voc, 4, 8192,
                                      EPI(scale=-1.0), FAKE, None, None, None) == vpa.VPA_ERR_INVALID


def test_module_covers_every_launch_entry_point():
    """_vpa_call marshals every entry point that enqueues work; the three
    host-only queries stay on ctypes."""
    host_only = {"vpa_stats_slots", "vpa_top_tokens_workspace", "vpa_last_error"}
    assert set(vpa.call().entries()) == set(vpa.SYMBOLS) - host_only


def test_module_rejects_bad_python_arguments():
    """Arguments the C types cannot hold raise before the library is called."""
    c = vpa.call()
    ok = (0x10000, vpa.VPA_BF16, 1000, 1000, 125, 8, 0, 256, None, 0, None, None, None, None, 0)
    assert c.vpa_top_tokens(*ok) == vpa.VPA_OK              # zero rows: nothing enqueued
    with pytest.raises(TypeError, match="takes 15 arguments"):
        c.vpa_top_tokens(*ok[:-1])
    with pytest.raises(OverflowError):                    # block is an int32
        c.vpa_top_tokens(*ok[:7], 1 << 31, *ok[8:])
    with pytest.raises(OverflowError):                    # addresses are unsigned
        c.vpa_top_tokens(-1, *ok[1:])
    with pytest.raises(TypeError):
        c.vpa_top_tokens(0x10000, vpa.VPA_BF16, 1000.0, *ok[3:])
    with pytest.raises(TypeError, match="epilogue"):
        c.vpa_top_tokens(*ok[:10], (None, 0), *ok[11:])
    with pytest.raises(TypeError):
        c.vpa_top_tokens(*ok[:10], (None, 0, "x"), *ok[11:])
    with pytest.raises(KeyError):
        c.bind("vpa_no_such_entry", 0x10000)
    with pytest.raises(ValueError):
        c.bind("vpa_top_tokens", 0)


def test_module_passes_scale_as_fp32():
    """A scale that rounds to zero as an fp32 is rejected as zero, as a C float
    argument would be."""
    c = vpa.call()
    args = (0x10000, vpa.VPA_BF16, 1000, 1000, 125, 8, 0, 256, None, 0, (None, 0, 1e-46),
            None, None, None, 0)
    assert c.vpa_top_tokens(*args) == vpa.VPA_ERR_INVALID
    assert "scale" in vpa.last_error()
    args = args[:10] + ((None, 0, 2.0 ** -149),) + args[11:]   # the least fp32 subnormal
    assert c.vpa_top_tokens(*args) == vpa.VPA_OK


def test_top_tokens_workspace_covers_both_cuts(lib):
    """vpa_top_tokens_workspace is the larger of the per-block statistics
    ([S][n][M]) and, when the sizes allow the chunked statistics of small
    bf16 batches, the chunk statistics ([n][ceil(V / 4096)])."""
    ws = lib.vpa_top_tokens_workspace
    assert ws(V(200064, 25008, 8), 1024, 8192) == 1024 * 49 * 8     # chunks: 49 > 8 * 4
    assert ws(V(200064, 25008, 8), 1025, 8192) == 1025 * 32 * 8     # past 1024 rows of 200064
    assert ws(V(200064, 25008, 8), 4096, 8192) == 4096 * 32 * 8
    assert ws(V(200063, 25008, 8), 64, 8192) == 64 * 32 * 8         # V not a multiple of 8
    assert ws(V(1000, 125, 8), 32768, 256) == 32768 * 16 * 8        # blocks need more
    assert ws(V(151936, 76032, 2), 1, 1024) == 2 * 75 * 8           # 1024-blocks need more


@pytest.mark.parametrize("dt,base,ld,need", [
    (vpa.VPA_BF16, FAKE, 152064, 32 * 38 * 8),                         # chunked statistics
    (vpa.VPA_F32, FAKE, 152064, 2 * 32 * 10 * 8),                      # fp32: per-block
    (vpa.VPA_BF16, ctypes.c_void_p(0x7F0000010008), 152064, 2 * 32 * 10 * 8),   # not 16-aligned
    (vpa.VPA_BF16, FAKE, 152068, 2 * 32 * 10 * 8),                     # ld not a multiple of 8
])
def test_top_tokens_picks_its_statistics_cut(lib, dt, base, ld, need):
    """Which statistics a call takes shows in the workspace bytes it asks for
    (every call here is rejected before anything is enqueued)."""
    voc = V(151936, 76032, 2)
    st = lib.vpa_top_tokens(base, dt, ld, voc, 32, 8192, FAKE, need - 8, None, FAKE, None, None,
                            None)
    assert st == vpa.VPA_ERR_INVALID
    assert f"smaller than {need} bytes" in vpa.last_error()
