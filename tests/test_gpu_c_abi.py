"""The C ABI from a C++ caller with no Python in the process
(kv_cache_compression_decode_amd/examples/rkv_c_example.cpp, built next to
librkv.so): one rkv_step on a small bf16 cache, checked by the program
itself on the host -- lengths, keep rows, compacted rows against the
original rows at the kept positions, an untriggered sequence untouched."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "kv_cache_compression_decode_amd", "rkv_c_example")


def test_c_program_runs_a_step():
    assert os.path.exists(EXE), "built with the library by kv_cache_compression_decode_amd.build"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
