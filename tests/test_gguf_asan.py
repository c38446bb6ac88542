"""The GGUF reader built with AddressSanitizer and UBSan (host code only, g++).

Compiles ggml_q2_dequant_amd/csrc/q2k_gguf.cpp with tests/gguf_asan_driver.cpp
and feeds it damaged and truncated versions of a valid file written as in
tests/test_gguf.py. CPU only; never needed on a GPU machine.
"""
import os

import numpy as np
import pytest

import synth
from test_gguf import BB, QK_K, _all_value_kinds, write_gguf

def test_reader_is_clean_under_address_sanitizer(tmp_path):
    """Build the reader with g++ -fsanitize=address (host code only) and feed it damaged files."""
    import shutil
    import subprocess
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    csrc = os.path.join(root, "ggml_q2_dequant_amd", "csrc")
    exe = str(tmp_path / "gguf_asan")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-I" + os.path.join(root, "include"), "-I" + csrc, os.path.join(csrc, "q2k_gguf.cpp"),
                    os.path.join(os.path.dirname(os.path.abspath(__file__)), "gguf_asan_driver.cpp"), "-o", exe],
                   check=True)
    good = bytearray(write_gguf(str(tmp_path / "g.gguf"), [("a", [QK_K], 10, 0), ("b", [QK_K, 2], 10, BB)],
                                kvs=_all_value_kinds(),
                                data=synth.random_blocks(np.random.Generator(np.random.PCG64(55)), 3).tobytes()))
    rng = np.random.Generator(np.random.PCG64(56))
    paths = []
    for i in range(300):
        bad = bytearray(good)
        if i % 3 == 0:
            bad = bad[:int(rng.integers(0, len(bad)))]
        else:
            for pos in rng.integers(0, len(bad), int(rng.integers(1, 8))):
                bad[pos] = int(rng.integers(0, 256))
        path = str(tmp_path / ("f%03d.gguf" % i))
        with open(path, "wb") as f:
            f.write(bad)
        paths.append(path)
    res = subprocess.run([exe, str(tmp_path / "g.gguf")] + paths, capture_output=True, text=True,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert res.returncode == 0, res.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
    assert res.stdout.startswith("opened ")
