"""The HBM read-ceiling probe (hbm_probe/vpa_probe.h, libvpa_probe.so): on the
CPU, its exports, header and argument checks; on the GPU, that one call reads
every byte of the read range exactly once (the XOR of the sink equals the
XOR of the range's 32-bit words, computed with numpy)."""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest
import torch

import hbm_probe as read_probe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "hbm_probe",
                      "vpa_probe.h")
FAKE = ctypes.c_void_p(0x10000)


def test_exports_every_declared_symbol():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(vpa_[a-z_]+)\s*\(", text)))
    assert set(names) == set(read_probe.SYMBOLS), names
    lb = read_probe.lib()
    for name in names:
        assert hasattr(lb, name), name


def test_header_is_plain_c_and_cxx(tmp_path):
    cc, cxx = shutil.which("gcc"), shutil.which("g++")
    if not cc or not cxx:
        pytest.skip("gcc/g++ not available")
    src = tmp_path / "h.c"
    src.write_text('#include "vpa_probe.h"\nint main(void) { return 0; }\n')
    for cmd in ([cc, "-std=c99", "-pedantic"], [cxx, "-std=c++11", "-pedantic", "-x", "c++"]):
        subprocess.run(cmd + ["-Wall", "-Wextra", "-Werror", "-I", os.path.dirname(HEADER),
                              "-fsyntax-only", str(src)], check=True)


def test_sizes():
    lb = read_probe.lib()
    assert lb.vpa_probe_read_bytes(-5) == 0
    assert lb.vpa_probe_read_bytes(4095) == 0
    assert lb.vpa_probe_read_bytes(4096) == 4096
    assert lb.vpa_probe_read_bytes(3 * 4096 + 17) == 3 * 4096
    assert lb.vpa_probe_read_bytes(1 << 40) == 1 << 40
    assert lb.vpa_probe_sink_words(0) == 0
    assert lb.vpa_probe_sink_words(512) == 512 * 256


def test_invalid_arguments_enqueue_nothing():
    """Every rejection happens before any HIP call, so no GPU is needed."""
    lb = read_probe.lib()
    assert lb.vpa_probe_read(None, 1 << 20, FAKE, 4, None) == -1
    assert lb.vpa_probe_read(ctypes.c_void_p(0x10008), 1 << 20, FAKE, 4, None) == -1
    assert lb.vpa_probe_read(FAKE, 4095, FAKE, 4, None) == -1
    assert lb.vpa_probe_read(FAKE, 1 << 20, None, 4, None) == -1
    assert lb.vpa_probe_read(FAKE, 1 << 20, ctypes.c_void_p(0x10002), 4, None) == -1
    assert lb.vpa_probe_read(FAKE, 1 << 20, FAKE, 0, None) == -1
    assert lb.vpa_probe_read(FAKE, 1 << 20, FAKE, (1 << 20) + 1, None) == -1


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes,n_wg", [
    (4096, 1),                       # one chunk, one workgroup (three idle wavefronts)
    (64 * 4096 + 100, 3),            # more chunks than wavefronts; a ragged tail left unread
    (37 * 4096, 64),                 # more wavefronts than chunks
    (48 << 20, None),                # the benchmark's grid, 2 workgroups per CU
])
def test_reads_every_byte_once(nbytes, n_wg):
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(nbytes)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=gen)
    buf = host.to(dev)
    n_wg = n_wg or read_probe.default_workgroups(dev)
    sink = read_probe.make_sink(dev, n_wg)
    sink.fill_(0x5A5A5A5A)
    got_bytes = read_probe.read(buf, sink, n_wg)
    torch.cuda.synchronize()
    assert got_bytes == nbytes // 4096 * 4096
    want = np.bitwise_xor.reduce(host[:got_bytes].numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want
